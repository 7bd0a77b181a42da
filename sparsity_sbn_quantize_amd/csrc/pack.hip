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

// Stage 1: block b sums |w| over rows [b*n_out/B, (b+1)*n_out/B) in fp64. When rows are
// contiguous (ld_w == K) and 16-byte aligned, the block's rows are one flat float4 range read
// with four loads in flight per thread into four accumulators, combined in a fixed order; the
// grid is fixed per shape, so the sum (and gamma) is the same on every run.
__global__ __launch_bounds__(kAbsmeanThreads) void absmean_partial(const float* __restrict__ w,
                                                                   int64_t n_out, int64_t K,
                                                                   int64_t ld_w, int vec4,
                                                                   double* __restrict__ partials) {
  __shared__ double red[kAbsmeanThreads / 64];
  const int64_t B = gridDim.x;
  const int64_t r0 = n_out * blockIdx.x / B, r1 = n_out * (blockIdx.x + 1) / B;
  double acc = 0.0;
  auto abs4 = [](const float4 f) -> double {
    return (double)fabsf(f.x) + (double)fabsf(f.y) + (double)fabsf(f.z) + (double)fabsf(f.w);
  };
  if (vec4 && ld_w == K) {
    const float4* base = reinterpret_cast<const float4*>(w + r0 * ld_w);
    const int64_t n4 = (r1 - r0) * (K >> 2);
    constexpr int kU = 4;
    double a[kU] = {0.0, 0.0, 0.0, 0.0};
    int64_t i = threadIdx.x;
    for (; i + (kU - 1) * kAbsmeanThreads < n4; i += kU * kAbsmeanThreads) {
      float4 f[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) f[u] = base[i + u * kAbsmeanThreads];
#pragma unroll
      for (int u = 0; u < kU; ++u) a[u] += abs4(f[u]);
    }
    for (; i < n4; i += kAbsmeanThreads) a[0] += abs4(base[i]);
    acc = (a[0] + a[1]) + (a[2] + a[3]);
  } else if (vec4) {
    const int64_t kv = K >> 2;
    for (int64_t r = r0; r < r1; ++r) {
      const float4* row = reinterpret_cast<const float4*>(w + r * ld_w);
      for (int64_t i = threadIdx.x; i < kv; i += kAbsmeanThreads) acc += abs4(row[i]);
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

// Stage 2: one block combines the partials in a fixed order and writes gamma. With structured
// outliers (osum != nullptr), the sum of their |w| (nos group sums, also in a fixed order) is
// taken off, so gamma is the absmean of the weights the ternary path sees.
__global__ __launch_bounds__(kAbsmeanThreads) void absmean_finalize(
    const double* __restrict__ partials, int num, double count, float* __restrict__ gamma,
    const double* __restrict__ osum, int64_t nos) {
  __shared__ double red[kAbsmeanThreads / 64];
  __shared__ double red2[kAbsmeanThreads / 64];
  double acc = 0.0;
  for (int i = threadIdx.x; i < num; i += kAbsmeanThreads) acc += partials[i];
  double s = block_sum_f64(acc, red);
  if (osum) {
    double acc2 = 0.0;
    for (int64_t i = threadIdx.x; i < nos; i += kAbsmeanThreads) acc2 += osum[i];
    s -= block_sum_f64(acc2, red2);
  }
  if (threadIdx.x == 0) gamma[0] = count > 0.0 ? (float)(s / count) : 0.0f;
}

// Keep mask of one m-group a[0..M): i is kept iff fewer than n group members precede it in the
// order (|w| descending, position ascending). Magnitudes compare as fp32 bit patterns. For each
// pair i < j exactly one precedes the other, so rank_i = #{j > i: a_j > a_i} + #{j < i: a_j >= a_i}
// is counted with one compare per pair.
template <int M>
__device__ __forceinline__ uint32_t keep_mask_group(const uint32_t* a, int n) {
  int rank[M];
#pragma unroll
  for (int i = 0; i < M; ++i) rank[i] = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) {
#pragma unroll
    for (int j = i + 1; j < M; ++j) {
      const int c = a[j] > a[i] ? 1 : 0;
      rank[i] += c;
      rank[j] += 1 - c;
    }
  }
  uint32_t keep = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) keep |= (rank[i] < n ? 1u : 0u) << i;
  return keep;
}

// One workgroup per fragment (16 rows x 256 K). Thread t handles 16 consecutive positions of one
// row: brick slot lane t / 4 (row t/4 % 16, brick t/64) and positions 16 (t % 4) .. +15 of that
// brick, so the four threads of a row read 64 contiguous weights and the workgroup writes the
// fragment's code words (4 bytes per thread) and mask halves (2 bytes per thread) as one
// contiguous block each. Padding rows and positions are written as zero.
// Sparse 2:4 form (FORM == kFormSparse24, M == 4): thread t = 4s + w covers lane s and word w of
// that lane's four (block b = w / 2, half h = w % 2): quad positions 128b + 32g + 16h .. +15 (g =
// s / 16). It computes half of the block's code word and half of its index word; the thread pair
// (h = 0, 1) exchanges halves, and thread h writes word 2b + h (codes, index), so the code plane
// is still written as one contiguous block. Its mask halves go to the mask plane's brick layout.
template <int M, int FORM>
__global__ __launch_bounds__(256) void pack_fragments(const float* __restrict__ w, int64_t ld_w,
                                                      int vec4, Layout L,
                                                      const float* __restrict__ gamma_p,
                                                      uint8_t* __restrict__ mask_plane,
                                                      uint8_t* __restrict__ code_plane,
                                                      uint32_t* __restrict__ flip_parts,
                                                      uint32_t* __restrict__ vc_parts,
                                                      const uint16_t* __restrict__ omask) {
  const int64_t frag = blockIdx.x;
  const int64_t rb = frag / L.quads, bq = frag % L.quads;
  const int tid = threadIdx.x;
  const int lane_slot = tid >> 2, word = tid & 3;
  const int64_t row = rb * 16 + (lane_slot & 15);
  constexpr bool kSp24 = FORM == kFormSparse24;
  // quad-relative first position of this thread's 16
  const int qpos = kSp24 ? 128 * (word >> 1) + 32 * (lane_slot >> 4) + 16 * (word & 1)
                         : kBrickK * (lane_slot >> 4) + 16 * word;
  const int64_t k0 = bq * kQuadK + qpos;
  const int cnt = row < L.n_out ? (int)max<int64_t>(0, min<int64_t>(16, L.K - k0)) : 0;
  // This thread's 16 keep bits in the mask plane; the previous pack's bits are loaded first, so the
  // load overlaps the weight loads.
  uint16_t* mp = reinterpret_cast<uint16_t*>(mask_plane) + frag * 256 + tid;
  if constexpr (kSp24) {
    // mask plane in brick layout: brick qpos / 64 of the quad, bits (qpos % 64) .. +15
    const int64_t mslot = (frag << 6) | ((lane_slot & 15) + 16 * (qpos >> 6));
    mp = reinterpret_cast<uint16_t*>(mask_plane) + mslot * 4 + ((qpos & 63) >> 4);
  }
  const uint32_t old_keep = L.has_mask ? (uint32_t)*mp : 0u;
  // Structured outliers: this thread's 16 outlier bits (same layout as its keep bits); those
  // positions read as 0 below.
  uint32_t obits = 0u;
  if (omask) {
    const int64_t oslot = (frag << 6) | ((lane_slot & 15) + 16 * (qpos >> 6));
    obits = omask[oslot * 4 + ((qpos & 63) >> 4)];
  }
  const float* wr = w + row * ld_w + k0;
  uint32_t u[16];
  if (vec4 && cnt == 16) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float4 f = reinterpret_cast<const float4*>(wr)[v];
      u[4 * v] = __float_as_uint(f.x);
      u[4 * v + 1] = __float_as_uint(f.y);
      u[4 * v + 2] = __float_as_uint(f.z);
      u[4 * v + 3] = __float_as_uint(f.w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) u[i] = i < cnt ? __float_as_uint(wr[i]) : 0u;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) u[i] = (obits >> i) & 1u ? 0u : u[i];
  const uint32_t half_bits = __float_as_uint(0.5f * gamma_p[0]);
  const int n = L.n;
  uint32_t a[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = u[i] & 0x7FFFFFFFu;
  uint32_t keep = 0;
#pragma unroll
  for (int g = 0; g < 16 / M; ++g) {
    uint32_t kg = (1u << M) - 1u;
    if (n < M) kg = keep_mask_group<M>(a + g * M, n);
    if (g * M < cnt) keep |= kg << (g * M);
  }
  // Ternary value of each kept position: |w| > gamma/2 (the rounding of |w|/gamma reaches 1).
  uint32_t nz = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) nz |= (a[i] > half_bits ? 1u : 0u) << i;
  const uint32_t nz_dense = nz;  // the codes of the dense (n = m) ternary weights
  nz &= keep;
  if constexpr (kSp24) {
    // slots 8h + 2q (lower kept) and 8h + 2q + 1 (higher kept) of group q of the 16 positions:
    // the two set bits of the group's keep nibble (none in padding groups: slots stay zero).
    // The code of position p is nz_p << sign_p (0, 1 = +1, 2 = -1).
    const int h = word & 1;
    uint32_t sgn = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) sgn |= (u[i] >> 31) << i;
    uint32_t cw = 0, iw = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t k4 = (keep >> (4 * q)) & 0xFu;
      const uint32_t lo = k4 ? (uint32_t)__builtin_ctz(k4) : 0u;
      const uint32_t hi = k4 ? 31u - (uint32_t)__builtin_clz(k4) : 0u;
      const uint32_t plo = 4 * q + lo, phi = 4 * q + hi;
      const uint32_t clo = k4 ? ((nz >> plo) & 1u) << ((sgn >> plo) & 1u) : 0u;
      const uint32_t chi = k4 ? ((nz >> phi) & 1u) << ((sgn >> phi) & 1u) : 0u;
      const int slot = 8 * h + 2 * q;
      cw |= (clo << sp24_code_bit(slot)) | (chi << sp24_code_bit(slot + 1));
      iw |= (lo << (2 * slot)) | (hi << (2 * slot + 2));
    }
    const int src = (int)(threadIdx.x & 63);
    const uint32_t ocw = (uint32_t)__shfl(cw, src ^ 1, 64);
    const uint32_t oiw = (uint32_t)__shfl(iw, src ^ 1, 64);
    reinterpret_cast<uint32_t*>(code_plane)[frag * 256 + tid] = h == 0 ? (cw | ocw) : (iw | oiw);
  } else if constexpr (FORM == kFormPositional) {
    uint32_t cw = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t c = ((nz >> i) & 1u) ? ((u[i] >> 31) ? 2u : 1u) : 0u;
      cw |= c << (8 * (i & 3) + 2 * (i >> 2));
    }
    reinterpret_cast<uint32_t*>(code_plane)[frag * 256 + tid] = cw;
  } else {
    // Kept form: this thread's kept codes in ascending position, then the brick's four pieces
    // are concatenated (each holds exactly 16n/M codes) by the thread of word 0.
    uint32_t bits = 0;
    int nb = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((keep >> i) & 1u) {
        const uint32_t c = ((nz >> i) & 1u) ? ((u[i] >> 31) ? 3u : 1u) : 0u;
        bits |= c << nb;
        nb += 2;
      }
    }
    const int piece = 32 * n / M;  // bits per 16 positions
    const int src = (int)(threadIdx.x & 63);
    const uint64_t b1 = (uint32_t)__shfl(bits, src + 1, 64);
    const uint64_t b2 = (uint32_t)__shfl(bits, src + 2, 64);
    const uint64_t b3 = (uint32_t)__shfl(bits, src + 3, 64);
    if (word == 0) {
      const uint64_t all = bits | (b1 << piece) | (b2 << (2 * piece)) | (b3 << (3 * piece));
      const int cbb = L.code_brick_bytes;
      uint8_t* dst = code_plane + ((frag << 6) | lane_slot) * cbb;
      for (int i = 0; i < cbb; ++i) dst[i] = (uint8_t)(all >> (8 * i));
    }
  }
  if (L.has_mask) {
    // Mask flips (Sparse-BitNet, Figure 3 (b), the mask flip rate r_t): keep bits that differ
    // from the previous pack's. Each wave's count goes to its own slot (no atomics, no barrier);
    // the slots are summed only when the count is asked for.
    *mp = (uint16_t)keep;
    const uint32_t sum = wave_sum_u32((uint32_t)__builtin_popcount((old_keep ^ keep) & 0xFFFFu));
    if ((tid & 63) == 0) flip_parts[frag * 4 + (tid >> 6)] = sum;
  }
  if (vc_parts) {
    // Variance correction: nonzero counts of the dense and of the n:m ternary codes, per wave.
    const uint32_t d = wave_sum_u32((uint32_t)__builtin_popcount(nz_dense));
    const uint32_t sp = wave_sum_u32((uint32_t)__builtin_popcount(nz));
    if ((tid & 63) == 0) {
      vc_parts[(frag * 4 + (tid >> 6)) * 2] = d;
      vc_parts[(frag * 4 + (tid >> 6)) * 2 + 1] = sp;
    }
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

// The 64 int8 codes of brick `brick` of row `row` (position i at byte i % 4 of dec[i / 4]) and
// its keep mask, for every code form.
__device__ void decode_brick(const Layout& L, const uint8_t* mask_plane, const uint8_t* code_plane,
                             int64_t row, int64_t brick, uint32_t mask[2], uint32_t dec[16]) {
  const int64_t slot = brick_slot(L, row, brick);
  uint32_t codes[4];
  load_brick(L, mask_plane, code_plane, slot, mask, codes);
  if (L.form == kFormSparse24) {
    // this brick's 64 positions are lane groups g0 and g0 + 1 of block b of its quad
    const int64_t q = brick >> 2;
    const int p0 = kBrickK * (int)(brick & 3);
    const int b = p0 >> 7, g0 = (p0 & 127) >> 5;
#pragma unroll
    for (int i = 0; i < 16; ++i) dec[i] = 0;
    for (int hh = 0; hh < 2; ++hh) {
      const int64_t s2 = (((row >> 4) * L.quads + q) << 6) | ((row & 15) + 16 * (g0 + hh));
      const uint32_t* w = reinterpret_cast<const uint32_t*>(code_plane + s2 * 16) + 2 * b;
      for (int j = 0; j < 16; ++j) {
        const int pos = 32 * hh + sp24_pos(w[1], j);
        const uint32_t v = (uint32_t)pos_value((w[0] >> sp24_code_bit(j)) & 3u) & 0xFFu;
        dec[pos >> 2] |= v << (8 * (pos & 3));
      }
    }
  } else if (L.positional) {
#pragma unroll
    for (int j = 0; j < 4; ++j) exp_word_to_i8(codes[j], dec + 4 * j);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) dec[i] = 0;
    decode_kept_brick(mask, codes, L.n, L.m, L.has_mask, dec);
  }
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
  uint32_t mask[2], dec[16];
  decode_brick(L, mask_plane, code_plane, row, brick, mask, dec);
  const int64_t k0 = brick * kBrickK;
  const int cnt = (int)min<int64_t>(kBrickK, L.K - k0);
  for (int i = 0; i < cnt; ++i) {
    const int64_t o = row * L.K + k0 + i;
    if (codes_out) codes_out[o] = (int8_t)((dec[i >> 2] >> (8 * (i & 3))) & 0xFFu);
    if (keep_out) keep_out[o] = L.has_mask ? (uint8_t)((mask[i >> 5] >> (i & 31)) & 1u) : 1;
  }
}

// Reference packed format export: per row, code bytes [code_row_bytes] and mask bytes
// [mask_row_bytes]. Every brick holds whole groups, so brick b's kept codes are the row stream's
// bytes [b*rcb, (b+1)*rcb) with rcb = 16n/m, and its mask the bytes [8b, 8b+8).
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
    const int rcb = 16 * L.n / L.m;
    const int64_t b0 = brick * rcb;
    const int cnt = (int)min<int64_t>(rcb, crb - b0);
    uint8_t* dst = code_out + row * crb + b0;
    if (L.form == kFormSparse24) {
      // 2:4: the brick's 32 kept codes are slots 0..15 of lane groups g0 and g0 + 1, in order
      const int64_t q = brick >> 2;
      const int p0 = kBrickK * (int)(brick & 3);
      const int b = p0 >> 7, g0 = (p0 & 127) >> 5;
      const int npos = (int)min<int64_t>(kBrickK, L.K - brick * kBrickK);
      for (int hh = 0; hh < 2 && 32 * hh < npos; ++hh) {
        const int64_t s2 = (((row >> 4) * L.quads + q) << 6) | ((row & 15) + 16 * (g0 + hh));
        const uint32_t cw = reinterpret_cast<const uint32_t*>(code_plane + s2 * 16)[2 * b];
        uint32_t bits = 0;
        for (int j = 0; j < 16; ++j)
          bits |= ref_code(pos_value((cw >> sp24_code_bit(j)) & 3u)) << (2 * j);
        const int nbytes = min(4, (npos - 32 * hh + 7) / 8);  // 8 positions -> one code byte
        for (int i = 0; i < nbytes && 4 * hh + i < cnt; ++i) dst[4 * hh + i] = (uint8_t)(bits >> (8 * i));
      }
    } else if (L.positional) {
      uint32_t mask[2], codes[4];
      load_brick(L, mask_plane, code_plane, slot, mask, codes);
      const int npos = (int)min<int64_t>(kBrickK, L.K - brick * kBrickK);
      uint32_t acc = 0;  // pending stream bits
      int nacc = 0, out = 0;
      for (int p = 0; p < npos; ++p) {
        const uint32_t kept = L.has_mask ? ((mask[p >> 5] >> (p & 31)) & 1u) : 1u;
        if (!kept) continue;
        const int bit = pos_bit(p);
        acc |= ref_code(pos_value((codes[bit >> 5] >> (bit & 31)) & 3u)) << nacc;
        nacc += 2;
        if (nacc == 8) {
          if (out < cnt) dst[out] = (uint8_t)acc;
          ++out;
          acc = 0;
          nacc = 0;
        }
      }
      if (nacc > 0 && out < cnt) dst[out] = (uint8_t)acc;
    } else {
      const uint8_t* src = code_plane + slot * L.code_brick_bytes;
      for (int i = 0; i < cnt; ++i) dst[i] = src[i];
    }
  }
  if (mask_out && L.has_mask) {
    const int64_t b0 = brick * 8;
    const int cnt = (int)min<int64_t>(8, mrb - b0);
    for (int i = 0; i < cnt; ++i) mask_out[row * mrb + b0 + i] = mask_plane[slot * 8 + i];
  }
}

__global__ void copy_gamma(const float* src, float* dst) { dst[0] = src[0]; }

// Compact plane from the code planes: one wave per fragment quad (rb * quads + q); lane l encodes
// brick 4q + l / 16 of row 16 rb + l % 16: its nonzero mask, and its signs into the slots of
// their groups. The lanes' sign bits are merged into the quad's bit stream in LDS (a lane's csb
// <= 64 bits span at most three words) and written out by the whole wave. Rows past n_out and
// bricks past K encode as zero.
__global__ __launch_bounds__(256) void build_compact(Layout L, const uint8_t* mask_plane,
                                                     const uint8_t* code_plane, int64_t nfq,
                                                     uint8_t* __restrict__ cplane) {
  __shared__ uint32_t sb[4][130];  // 2 * 64 words of signs, +2 for the last lane's spill
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t fq = (int64_t)blockIdx.x * 4 + wave;
  const int S = L.csb;
  for (int i = lane; i < 130; i += 64) sb[wave][i] = 0u;
  __syncthreads();
  uint32_t nzm[2] = {0u, 0u};
  if (fq < nfq) {
    const int64_t row = (fq / L.quads) * 16 + (lane & 15);
    const int64_t brick = (fq % L.quads) * kFragBricks + (lane >> 4);
    unsigned long long sg = 0ull;
    if (row < L.n_out) {
      uint32_t mask[2], dec[16];
      decode_brick(L, mask_plane, code_plane, row, brick, mask, dec);
      int j = 0;  // nonzero codes seen so far in the current group
      for (int p = 0; p < kBrickK; ++p) {
        if (p % L.m == 0) j = 0;
        const uint32_t v = (dec[p >> 2] >> (8 * (p & 3))) & 0xFFu;
        if (v != 0u) {
          nzm[p >> 5] |= 1u << (p & 31);
          if (v == 0xFFu) sg |= 1ull << ((p / L.m) * L.n + j);
          ++j;
        }
      }
    }
    const int bit = lane * S;
    const int d = bit >> 5, sh = bit & 31;
    const uint32_t lo = (uint32_t)sg, hi = (uint32_t)(sg >> 32);
    const uint32_t w0 = lo << sh;
    const uint32_t w1 = sh ? ((hi << sh) | (lo >> (32 - sh))) : hi;
    const uint32_t w2 = sh ? (hi >> (32 - sh)) : 0u;
    if (w0) atomicOr(&sb[wave][d], w0);
    if (w1) atomicOr(&sb[wave][d + 1], w1);
    if (w2) atomicOr(&sb[wave][d + 2], w2);
  }
  __syncthreads();
  if (fq < nfq) {
    uint8_t* dst = cplane + fq * compact_quad_bytes(S);
    reinterpret_cast<uint2*>(dst)[lane] = make_uint2(nzm[0], nzm[1]);
    uint32_t* sd = reinterpret_cast<uint32_t*>(dst + kCompactMaskBytes);
    for (int i = lane; i < 2 * S; i += 64) sd[i] = sb[wave][i];
  }
}

// Export of the compact plane as per-row bit streams: group g at bits [g (m + n), (g+1) (m + n)),
// its m nonzero-mask bits first, then its n sign slots; LSB first, rows padded to a byte. One
// thread per output byte, each bit read from the plane.
__global__ __launch_bounds__(256) void export_compact(Layout L, const uint8_t* cplane, int64_t crb,
                                                      uint8_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= L.n_out * crb) return;
  const int64_t row = idx / crb, byte = idx % crb;
  const int gbits = L.m + L.n;
  const int64_t total = (L.K / L.m) * gbits;
  const int S = L.csb;
  uint32_t v = 0u;
  for (int t = 0; t < 8; ++t) {
    const int64_t B = byte * 8 + t;
    if (B >= total) break;
    const int64_t g = B / gbits;
    const int p = (int)(B % gbits);
    const int64_t pos0 = g * L.m, brick = pos0 >> 6;
    const int lane = (int)((row & 15) | ((brick & 3) << 4));
    const uint32_t* frag = reinterpret_cast<const uint32_t*>(
        cplane + ((row >> 4) * L.quads + (brick >> 2)) * compact_quad_bytes(S));
    uint32_t bv;
    if (p < L.m) {
      const int pb = (int)(pos0 & 63) + p;
      bv = (frag[2 * lane + (pb >> 5)] >> (pb & 31)) & 1u;
    } else {
      const int gl = (int)((pos0 & 63) / L.m);
      const int64_t sbit = (int64_t)lane * S + gl * L.n + (p - L.m);
      bv = (frag[kCompactMaskBytes / 4 + (sbit >> 5)] >> (sbit & 31)) & 1u;
    }
    v |= bv << t;
  }
  out[row * crb + byte] = (uint8_t)v;
}
// Transposed code plane, read by the data-gradient matmul, whose reduction runs over the rows:
// for every 16 columns cb and 128 rows rq, 64 lanes x 8 bytes at slot (cb * rq_count + rq) * 64
// + lane. Lane l = c + 16 g holds column 16 cb + c of rows 128 rq + 32 g + (0..31); its word h
// (0, 1) holds row 32 g + 16 h + 8 s + 2 p + e (s, e in {0, 1}, p in 0..3) at bits
// 2 p + 8 s + 16 e, as 2-bit codes 0 = 0, 1 = +1, 2 = -1. One workgroup per 128 rows x 256
// columns: its 512 bricks are decoded into LDS as 2-bit codes (row-major, 16 positions per
// word), then every thread assembles 8 words of 8 columns. Rows past n_out are zero.
__global__ __launch_bounds__(256) void transpose_codes(Layout L, const uint8_t* mask_plane,
                                                       const uint8_t* code_plane,
                                                       int64_t rq_count,
                                                       uint32_t* __restrict__ tplane) {
  __shared__ uint32_t cw[128][17];  // row x 16 code words (+1 against bank conflicts)
  const int64_t rq = blockIdx.x / L.quads, q = blockIdx.x % L.quads;
  const int tid = threadIdx.x;
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i, rl = idx >> 2, b = idx & 3;
    const int64_t row = rq * 128 + rl;
    uint32_t w4[4] = {0u, 0u, 0u, 0u};
    if (row < L.n_out) {
      uint32_t mask[2], dec[16];
      decode_brick(L, mask_plane, code_plane, row, q * kFragBricks + b, mask, dec);
      for (int j = 0; j < kBrickK; ++j) {
        const uint32_t v = (dec[j >> 2] >> (8 * (j & 3))) & 0xFFu;
        w4[j >> 4] |= (v == 0xFFu ? 2u : v) << (2 * (j & 15));
      }
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) cw[rl][4 * b + w] = w4[w];
  }
  __syncthreads();
  const int task = tid >> 1, half = tid & 1;
  const int cbl = task >> 3, g = (task >> 1) & 3, h = task & 1;
  uint32_t rw[16];
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) rw[rr] = cw[32 * g + 16 * h + rr][cbl];
  const int64_t cb = q * 16 + cbl;
  uint32_t* const dst = tplane + (cb * rq_count + rq) * 128;
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) {
    const int c = 8 * half + cc;
    uint32_t out = 0;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)  // rr = 8 s + 2 p + e
      out |= ((rw[rr] >> (2 * c)) & 3u) << (2 * ((rr >> 1) & 3) + 8 * (rr >> 3) + 16 * (rr & 1));
    dst[(c + 16 * g) * 2 + h] = out;
  }
}

// Variance correction ("From 2:4 to 8:16 sparsity patterns in LLMs for Outliers and Weights with
// Variance Correction", the method summary: the remaining weights are rescaled back to the dense
// variance). The weights the matmul uses are gamma * codes, whose mean square is gamma^2 times the
// share of nonzero codes, so the factor is sqrt(nonzero dense codes / nonzero n:m codes) and the
// output scale is gamma_out = fl32(gamma * sqrt(nd / ns)) (gamma when ns == 0). One workgroup.
__global__ __launch_bounds__(1024) void vc_finalize(const uint32_t* __restrict__ parts, int64_t num,
                                                    const float* __restrict__ gamma,
                                                    float* __restrict__ gamma_out) {
  __shared__ unsigned long long red[2][16];
  unsigned long long d = 0, sp = 0;
  for (int64_t i = threadIdx.x; i < num; i += 1024) {
    d += parts[2 * i];
    sp += parts[2 * i + 1];
  }
  for (int o = 32; o >= 1; o >>= 1) {
    d += __shfl_xor(d, o, 64);
    sp += __shfl_xor(sp, o, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = d;
    red[1][threadIdx.x >> 6] = sp;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long td = 0, ts = 0;
    for (int i = 0; i < 16; ++i) {
      td += red[0][i];
      ts += red[1][i];
    }
    const double g = (double)gamma[0];
    gamma_out[0] = ts == 0 ? gamma[0] : (float)(g * sqrt((double)td / (double)ts));
  }
}

// Sum of the per-wave flip counts of the last pack (one workgroup; num may be 0).
__global__ __launch_bounds__(1024) void sum_flips(const uint32_t* __restrict__ parts, int64_t num,
                                                  unsigned long long* __restrict__ out) {
  __shared__ unsigned long long red[16];
  unsigned long long acc = 0;
  for (int64_t i = threadIdx.x; i < num; i += 1024) acc += parts[i];
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long t = 0;
    for (int i = 0; i < 16; ++i) t += red[i];
    out[0] = t;
  }
}

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
  const bool outl = h->outlier_k > 0 && L.n_out > 0;
  if (outl) {
    hipError_t e = launch_outlier_select(w, ld_w, h, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(absmean_finalize, dim3(1), dim3(kAbsmeanThreads), 0, s, h->partials,
                     L.n_out > 0 ? h->num_partials : 0, (double)L.n_out * (double)L.K, h->gamma,
                     outl ? h->osum : nullptr,
                     outl ? (L.n_out * (L.K >> 8) + 255) / 256 : (int64_t)0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || L.n_out == 0) return e;
  const dim3 grid((unsigned)(L.row_blocks_pad * L.quads));
  uint32_t* const vc = h->vc ? h->vc_parts : nullptr;
#define SBN_PACK(MM, FF)                                                                      \
  hipLaunchKernelGGL((pack_fragments<MM, FF>), grid, dim3(256), 0, s, w, ld_w, vec4, L, h->gamma, \
                     h->mask, h->codes, h->flip_parts, vc,                                   \
                     outl ? reinterpret_cast<const uint16_t*>(h->omask) : nullptr)
  if (L.form == kFormSparse24) {
    SBN_PACK(4, kFormSparse24);
  } else if (L.m == 4) {
    if (L.positional) SBN_PACK(4, kFormPositional); else SBN_PACK(4, kFormKept);
  } else if (L.m == 8) {
    if (L.positional) SBN_PACK(8, kFormPositional); else SBN_PACK(8, kFormKept);
  } else {
    if (L.positional) SBN_PACK(16, kFormPositional); else SBN_PACK(16, kFormKept);
  }
#undef SBN_PACK
  if (h->compact) {
    const int64_t nfq = L.row_blocks_pad * L.quads;
    hipLaunchKernelGGL(build_compact, dim3((unsigned)((nfq + 3) / 4)), dim3(256), 0, s, L, h->mask,
                       h->codes, nfq, h->cplane);
  }
  if (h->vc) {
    hipLaunchKernelGGL(vc_finalize, dim3(1), dim3(1024), 0, s, h->vc_parts,
                       L.row_blocks_pad * L.quads * 4, h->gamma, h->gamma_vc);
  }
  return hipGetLastError();
}

// Rank encoding (export): per group, the rank of its keep mask in the combinatorial number system
// (colex order of the kept positions: sum over the i-th kept position c of C(c, i), i from 1),
// R = ceil(log2 C(m, n)) bits, then its n kept codes' low two bits by ascending position; rows LSB
// first, padded to a byte. One thread per row and 128 positions (two bricks): its 128 / m groups
// take (128 / m)(R + 2n) bits, a whole number of bytes for m in {4, 8, 16}, so threads write
// disjoint bytes and the last thread of a row writes the padding.
namespace {

// C(c, i) for c < 16, i <= 16 (Pascal's rule), in constant memory: the rank is a sum of table reads.
struct BinomTable {
  uint16_t v[16][17];
};
constexpr BinomTable make_binom_table() {
  BinomTable t{};
  for (int c = 0; c < 16; ++c) {
    t.v[c][0] = 1;
    for (int i = 1; i <= 16; ++i) t.v[c][i] = c == 0 ? 0 : (uint16_t)(t.v[c - 1][i - 1] + t.v[c - 1][i]);
  }
  return t;
}
__constant__ BinomTable kBinom = make_binom_table();

__device__ __forceinline__ uint32_t binom16(int c, int i) { return kBinom.v[c][i]; }

__global__ __launch_bounds__(256) void export_rank(Layout L, const uint8_t* mask_plane,
                                                   const uint8_t* code_plane, int R,
                                                   int64_t row_bytes, uint8_t* __restrict__ out) {
  const int64_t nchunks = (L.K + 127) / 128;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= L.n_out * nchunks) return;
  const int64_t row = idx / nchunks, chunk = idx % nchunks;
  const int m = L.m, n = L.n, per = R + 2 * n;
  uint8_t* dst = out + row * row_bytes + chunk * (128 / m) * per / 8;
  uint64_t acc = 0;
  int nb = 0;
  auto put = [&](uint32_t v, int bits) {  // bits <= 16
    acc |= (uint64_t)v << nb;
    nb += bits;
    while (nb >= 8) {
      *dst++ = (uint8_t)acc;
      acc >>= 8;
      nb -= 8;
    }
  };
  for (int b = 0; b < 2; ++b) {
    const int64_t brick = chunk * 2 + b;
    const int64_t k0 = brick * kBrickK;
    if (k0 >= L.K) break;
    uint32_t mask[2], dec[16];
    decode_brick(L, mask_plane, code_plane, row, brick, mask, dec);
    const int groups = (int)(min<int64_t>(kBrickK, L.K - k0) / m);
    for (int g = 0; g < groups; ++g) {
      uint32_t r = 0u;
      int i = 0;
      for (int p = 0; p < m; ++p) {
        const int pos = g * m + p;
        if (!L.has_mask || ((mask[pos >> 5] >> (pos & 31)) & 1u)) r += binom16(p, ++i);
      }
      put(r, R);
      for (int p = 0; p < m; ++p) {
        const int pos = g * m + p;
        if (!L.has_mask || ((mask[pos >> 5] >> (pos & 31)) & 1u))
          put((dec[pos >> 2] >> (8 * (pos & 3))) & 3u, 2);
      }
    }
  }
  if (nb > 0) *dst = (uint8_t)acc;  // the row's last byte: padding bits are zero
}

}  // namespace

int rank_bits(int n, int m) {
  uint64_t c = 1;
  for (int j = 1; j <= n; ++j) c = c * (uint64_t)(m - n + j) / (uint64_t)j;  // C(m, n)
  int b = 0;
  while ((uint64_t{1} << b) < c) ++b;
  return b;
}

hipError_t launch_export_rank(const sbn_packed* h, uint8_t* out, hipStream_t s) {
  const Layout& L = h->L;
  const int64_t total = L.n_out * ((L.K + 127) / 128);
  if (total == 0) return hipSuccess;
  const int R = rank_bits((int)L.n, (int)L.m);
  const int64_t row_bytes = ((L.K / L.m) * (R + 2 * L.n) + 7) / 8;
  hipLaunchKernelGGL(export_rank, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, L,
                     h->mask, h->codes, R, row_bytes, out);
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
  if (gamma) hipLaunchKernelGGL(copy_gamma, dim3(1), dim3(1), 0, s, h->gamma_out(), gamma);
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

namespace sbn {
hipError_t launch_export_compact(const sbn_packed* h, uint8_t* out, hipStream_t s) {
  const Layout& L = h->L;
  const int64_t total = L.n_out * (int64_t)h->compact_row_bytes;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(export_compact, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, L,
                     h->cplane, (int64_t)h->compact_row_bytes, out);
  return hipGetLastError();
}

hipError_t launch_transpose_codes(const sbn_packed* h, hipStream_t s) {
  const Layout& L = h->L;
  if (h->rq_count == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_codes, dim3((unsigned)(h->rq_count * L.quads)), dim3(256), 0, s, L,
                     h->mask, h->codes, h->rq_count, h->tplane);
  return hipGetLastError();
}

hipError_t launch_sum_flips(const sbn_packed* h, uint64_t* out, hipStream_t s) {
  const Layout& L = h->L;
  const int64_t num = (L.has_mask && L.n_out > 0) ? L.row_blocks_pad * L.quads * 4 : 0;
  hipLaunchKernelGGL(sum_flips, dim3(1), dim3(1024), 0, s, h->flip_parts, num,
                     reinterpret_cast<unsigned long long*>(out));
  return hipGetLastError();
}
}  // namespace sbn
