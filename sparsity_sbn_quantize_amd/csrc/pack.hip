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

#include <algorithm>
#include <type_traits>

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
    const double* __restrict__ osum, int64_t nos, uint32_t* __restrict__ pack_gen) {
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
  if (threadIdx.x == 0) {
    gamma[0] = count > 0.0 ? (float)(s / count) : 0.0f;
    pack_gen[0] += 1u;  // one more pack of the handle (the transposed plane is now stale)
  }
}

// Keep mask of one m-group a[0..M) by rank counting (used for M = 4): i is kept iff fewer than n
// group members precede it in the order (|w| descending, position ascending). Magnitudes compare
// as fp32 bit patterns. For each pair i < j exactly one precedes the other, so
// rank_i = #{j > i: a_j > a_i} + #{j < i: a_j >= a_i} is counted with one compare per pair.
template <int M>
__device__ __forceinline__ uint32_t keep_mask_rank(const uint32_t* a, int n) {
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

// Compare-exchange to descending order, and the 19-comparator sorting network for 8 values.
__device__ __forceinline__ void cx_desc(uint32_t& a, uint32_t& b) {
  const uint32_t hi = max(a, b), lo = min(a, b);
  a = hi;
  b = lo;
}
__device__ __forceinline__ void sort8_desc(uint32_t* v) {
  cx_desc(v[0], v[2]); cx_desc(v[1], v[3]); cx_desc(v[4], v[6]); cx_desc(v[5], v[7]);
  cx_desc(v[0], v[4]); cx_desc(v[1], v[5]); cx_desc(v[2], v[6]); cx_desc(v[3], v[7]);
  cx_desc(v[0], v[1]); cx_desc(v[2], v[3]); cx_desc(v[4], v[5]); cx_desc(v[6], v[7]);
  cx_desc(v[2], v[4]); cx_desc(v[3], v[5]);
  cx_desc(v[1], v[4]); cx_desc(v[3], v[6]);
  cx_desc(v[1], v[2]); cx_desc(v[3], v[4]); cx_desc(v[5], v[6]);
}

// Keep mask of one group of M = 8 or 16 by selection (the same mask as keep_mask_rank, about a
// third of its ALU work for M = 16): v = the n-th largest magnitude (M = 8: one sorted group;
// M = 16: the two sorted halves A, B give v = max over splits i of min(A[i-1], B[n-i-1]), the
// n-th largest of a union of two sorted lists). Every magnitude above v is kept, and of those
// equal to v the lowest positions, as many as are still missing (ties go to the lower index).
template <int M>
__device__ __forceinline__ uint32_t keep_mask_select(const uint32_t* a, int n) {
  uint32_t A[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) A[i] = a[i];
  sort8_desc(A);
  uint32_t v;
  if constexpr (M == 8) {
    v = A[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) v = n - 1 == i ? A[i] : v;
  } else {
    uint32_t B[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) B[i] = a[8 + i];
    sort8_desc(B);
    v = 0;
#pragma unroll
    for (int i = 0; i <= 8; ++i) {
      const int j = n - i;
      const uint32_t x = i > 0 ? A[i - 1] : 0xFFFFFFFFu;
      const uint32_t y = j > 0 && j <= 8 ? B[j - 1] : 0xFFFFFFFFu;
      v = max(v, j >= 0 && j <= 8 ? min(x, y) : 0u);
    }
  }
  uint32_t gt = 0, ge = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    gt |= (a[i] > v ? 1u : 0u) << i;
    ge |= (a[i] >= v ? 1u : 0u) << i;
  }
  const uint32_t eq = ge & ~gt;
  const int r = n - __builtin_popcount(gt);  // 1 <= r <= popcount(eq)
  if (__builtin_popcount(eq) == r) return gt | eq;
  uint32_t e = eq, kept = 0;
  for (int j = 0; j < r; ++j) {
    const uint32_t low = e & (~e + 1u);
    kept |= low;
    e ^= low;
  }
  return gt | kept;
}

template <int M>
__device__ __forceinline__ uint32_t keep_mask_group(const uint32_t* a, int n) {
  if constexpr (M == 4) {
    return keep_mask_rank<M>(a, n);
  } else {
    return keep_mask_select<M>(a, n);
  }
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

// ---------------------------------------------------------------------------------------------
// Lean piece encoder and the single-pass re-pack.
//
// The same thread mapping as pack_fragments (one workgroup per fragment, thread t takes 16
// consecutive positions of one row), with the keep mask and the codes built for fixed n:m
// patterns (2:4, 4:8, 6:8, 8:16 and n = m) with fewer vector instructions: the n-th largest
// magnitude of a group comes from a sorting network without run-time selects, the 16 predicate
// bits of a thread are shifted in one per compare (the compare's lane mask is the carry of an
// add), and the positional code word is two bit spreads of the nonzero and sign masks.
//
// Single pass. gamma must be known before a code can be written, so the first pack of a handle
// reads the latent weights twice (absmean, then the codes). A re-pack instead takes the previous
// pack's gamma g' and the bracket [T_lo, T_hi] = g'/2 (1 -+ 2^-7) around its threshold: every
// kept magnitude above T_hi is nonzero and every one at or below T_lo is zero for any new
// threshold inside the bracket, so one read writes the codes, the keep mask and gamma's partial
// sums, and lists the pieces that hold a kept magnitude inside the bracket (their codes are
// written as zero there). After the absmean is finalized, pack_fix checks that the new threshold
// lies in the bracket and sets the listed pieces' nonzero codes; if it does not (gamma moved by
// more than 2^-7), or a fragment listed more pieces than it has room for, pack_fix rewrites those
// fragments' codes from the latent weights and the stored keep bits. The result is the same
// planes as the two-pass pack in every case.
constexpr float kBandHalfWidth = 0.0078125f;  // 2^-7

// acc * 2 + predicate: a compare into VCC and an add with carry (one vector instruction each).
__device__ __forceinline__ uint32_t shl_gt(uint32_t acc, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_cmp_gt_u32_e32 vcc, %1, %2\n\tv_addc_co_u32_e32 %0, vcc, %3, %3, vcc"
      : "=v"(r) : "v"(a), "v"(b), "v"(acc) : "vcc");
  return r;
}
__device__ __forceinline__ uint32_t shl_ge(uint32_t acc, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_cmp_ge_u32_e32 vcc, %1, %2\n\tv_addc_co_u32_e32 %0, vcc, %3, %3, vcc"
      : "=v"(r) : "v"(a), "v"(b), "v"(acc) : "vcc");
  return r;
}
__device__ __forceinline__ uint32_t shl_neg(uint32_t acc, uint32_t x) {
  uint32_t r;
  asm("v_cmp_gt_i32_e32 vcc, 0, %1\n\tv_addc_co_u32_e32 %0, vcc, %2, %2, vcc"
      : "=v"(r) : "v"(x), "v"(acc) : "vcc");
  return r;
}

// Position whose bit lands at bit k of a transposed mask: bit 4b + a holds position 4a + b, the
// order of the positional code word (position i at bits 8 (i & 3) + 2 (i >> 2)).
__device__ __forceinline__ constexpr int tpos(int k) { return 4 * (k & 3) + (k >> 2); }
// Natural 16-bit mask (bit i = position i) to the transposed order.
__device__ __forceinline__ uint32_t transpose4x4(uint32_t x) {
  uint32_t t = (x ^ (x >> 3)) & 0x0A0Au;
  x ^= t ^ (t << 3);
  t = (x ^ (x >> 6)) & 0x00CCu;
  x ^= t ^ (t << 6);
  return x;
}
// Bit k to bit 2k.
__device__ __forceinline__ uint32_t spread2(uint32_t x) {
  x = (x | (x << 8)) & 0x00FF00FFu;
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  x = (x | (x << 2)) & 0x33333333u;
  x = (x | (x << 1)) & 0x55555555u;
  return x;
}

// The patterns with a lean encoder; N == M stands for every dense pattern.
__host__ __device__ constexpr bool lean_pattern(int n, int m) {
  return n == m || (m == 4 && n == 2) || (m == 8 && (n == 4 || n == 6)) || (m == 16 && n == 8);
}

// The n-th largest magnitude of each group (16 / M groups of the thread's 16).
template <int M, int N>
__device__ __forceinline__ void group_nth(const uint32_t* a, uint32_t* v) {
  if constexpr (M == 4 && N == 2) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t* x = a + 4 * g;
      const uint32_t h01 = max(x[0], x[1]), l01 = min(x[0], x[1]);
      const uint32_t h23 = max(x[2], x[3]), l23 = min(x[2], x[3]);
      v[g] = max(min(h01, h23), max(l01, l23));
    }
  } else if constexpr (M == 8) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      uint32_t s[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = a[8 * g + i];
      sort8_desc(s);
      v[g] = s[N - 1];
    }
  } else {
    static_assert(M == 16, "lean patterns");
    uint32_t A[8], B[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      A[i] = a[i];
      B[i] = a[8 + i];
    }
    sort8_desc(A);
    sort8_desc(B);
    // n-th largest of the union of two descending lists: max over the split i (i from A, n - i
    // from B) of the smaller of the two last elements taken
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i <= 8; ++i) {
      const int j = N - i;
      if (j < 0 || j > 8) continue;
      const uint32_t x = i > 0 ? A[i - 1] : 0xFFFFFFFFu;
      const uint32_t y = j > 0 ? B[j - 1] : 0xFFFFFFFFu;
      r = max(r, min(x, y));
    }
    v[0] = r;
  }
}

// Keep mask of the thread's 16 positions (bit i = position i), the rule of keep_mask_group: the
// n largest magnitudes of each group, equal magnitudes to the lower position. Without ties the
// positions at or above each group's n-th largest are exactly n per group; otherwise the group
// takes those above it and the lowest positions equal to it. Groups starting at or past cnt are
// empty. v receives the groups' n-th largest magnitudes.
template <int M, int N>
__device__ __forceinline__ uint32_t lean_keep(const uint32_t* a, int cnt, uint32_t* v) {
  constexpr int G = 16 / M;
  uint32_t keep;
  if constexpr (N == M) {
    keep = 0xFFFFu;
  } else {
    group_nth<M, N>(a, v);
    uint32_t ge = 0;
#pragma unroll
    for (int i = 15; i >= 0; --i) ge = shl_ge(ge, a[i], v[i / M]);
    keep = ge;
    if (__builtin_popcount(ge) != G * N) {
      keep = 0;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        uint32_t gt = 0;
#pragma unroll
        for (int i = 0; i < M; ++i) gt |= (a[g * M + i] > v[g] ? 1u : 0u) << i;
        uint32_t eq = ((ge >> (g * M)) & ((1u << M) - 1u)) & ~gt;
        uint32_t kept = gt;
        for (int r = N - __builtin_popcount(gt); r > 0; --r) {
          const uint32_t low = eq & (~eq + 1u);
          kept |= low;
          eq ^= low;
        }
        keep |= kept << (g * M);
      }
    }
  }
  if (cnt < 16) {
    uint32_t live = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) live |= (g * M < cnt ? (1u << M) - 1u : 0u) << (g * M);
    keep &= live;
  }
  return keep;
}

// Where a thread's 16 positions live: its fragment, row and K range, and its slots in the planes.
struct PieceAt {
  int64_t row, k0;
  int cnt;        // positions inside the weight (0 for padding rows)
  int lane_slot, word;
};
template <int FORM>
__device__ __forceinline__ PieceAt piece_at(const Layout& L, int64_t frag, int tid) {
  PieceAt p;
  const int64_t rb = frag / L.quads, bq = frag % L.quads;
  p.lane_slot = tid >> 2;
  p.word = tid & 3;
  p.row = rb * 16 + (p.lane_slot & 15);
  const int qpos = FORM == kFormSparse24
                       ? 128 * (p.word >> 1) + 32 * (p.lane_slot >> 4) + 16 * (p.word & 1)
                       : kBrickK * (p.lane_slot >> 4) + 16 * p.word;
  p.k0 = bq * kQuadK + qpos;
  p.cnt = p.row < L.n_out ? (int)max<int64_t>(0, min<int64_t>(16, L.K - p.k0)) : 0;
  return p;
}
// The thread's 16 keep bits in the mask plane (brick layout for the 2:4 form).
template <int FORM>
__device__ __forceinline__ uint16_t* piece_mask(uint8_t* mask_plane, int64_t frag, int tid,
                                                const PieceAt& p) {
  if constexpr (FORM == kFormSparse24) {
    const int qpos = 128 * (p.word >> 1) + 32 * (p.lane_slot >> 4) + 16 * (p.word & 1);
    const int64_t mslot = (frag << 6) | ((p.lane_slot & 15) + 16 * (qpos >> 6));
    return reinterpret_cast<uint16_t*>(mask_plane) + mslot * 4 + ((qpos & 63) >> 4);
  } else {
    return reinterpret_cast<uint16_t*>(mask_plane) + frag * 256 + tid;
  }
}
__device__ __forceinline__ void load_piece(const float* w, int64_t ld_w, int vec4,
                                           const PieceAt& p, uint32_t* u) {
  const float* wr = w + p.row * ld_w + p.k0;
  if (vec4 && p.cnt == 16) {
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
    for (int i = 0; i < 16; ++i) u[i] = i < p.cnt ? __float_as_uint(wr[i]) : 0u;
  }
}

// Writes the thread's code word from its keep mask, the nonzero cut (a kept magnitude above it
// is nonzero) and the signs. Positional: one word per thread. 2:4: the thread pair (h = 0, 1)
// exchanges halves and thread h writes word 2b + h (codes, index). All 64 lanes of the wave call
// it together.
template <int FORM>
__device__ __forceinline__ void lean_codes(const uint32_t* u, const uint32_t* a, uint32_t keep,
                                           uint32_t cut, uint32_t* code_word, int word) {
  if constexpr (FORM == kFormPositional) {
    uint32_t nzt = 0, sgt = 0;
#pragma unroll
    for (int k = 15; k >= 0; --k) {
      nzt = shl_gt(nzt, a[tpos(k)], cut);
      sgt = shl_neg(sgt, u[tpos(k)]);
    }
    const uint32_t nt = nzt & transpose4x4(keep);
    *code_word = spread2(nt) + spread2(nt & sgt);
  } else {
    static_assert(FORM == kFormSparse24, "lean forms");
    uint32_t nz = 0, sgn = 0;
#pragma unroll
    for (int i = 15; i >= 0; --i) {
      nz = shl_gt(nz, a[i], cut);
      sgn = shl_neg(sgn, u[i]);
    }
    nz &= keep;
    // 2-bit code of every position (bits 2i, 2i + 1: 0, 1 = +1, 2 = -1), then per group the
    // codes at its lowest and highest kept positions (none in padding groups: slots stay zero)
    const uint32_t cn = spread2(nz) + spread2(nz & sgn);
    // built for half h = 0 (constant shifts); half 1's slots are 8 further on, which moves the
    // code bits up by 4 and the index bits up by 16
    const int h = word & 1;
    uint32_t cw = 0, iw = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t k4 = (keep >> (4 * q)) & 0xFu;
      // lowest and highest kept position (0 and 0 in padding groups, where k4 == 0)
      const uint32_t lo = (uint32_t)__builtin_ctz(k4 | 0x10u) & 3u;
      const uint32_t hi = 31u - (uint32_t)__builtin_clz(k4 | 1u);
      const uint32_t clo = (cn >> (8 * q + 2 * lo)) & 3u;  // 0 when k4 == 0 (nz is 0 there)
      const uint32_t chi = (cn >> (8 * q + 2 * hi)) & 3u;
      cw |= (clo << sp24_code_bit(2 * q)) | (chi << sp24_code_bit(2 * q + 1));
      iw |= (lo << (4 * q)) | (hi << (4 * q + 2));
    }
    cw <<= 4 * h;
    iw <<= 16 * h;
    const int src = (int)(threadIdx.x & 63);
    const uint32_t ocw = (uint32_t)__shfl(cw, src ^ 1, 64);
    const uint32_t oiw = (uint32_t)__shfl(iw, src ^ 1, 64);
    *code_word = h == 0 ? (cw | ocw) : (iw | oiw);
  }
}

// Workspace of the single pass: gamma's partial sum per fragment, a record per fragment (the
// number of pieces it listed, then up to kBandSegCap piece indices), and the bracket [T_lo, T_hi]
// the pass used (as fp32 bit patterns).
struct BandWs {
  double* part;
  uint8_t* seg;
  uint32_t* lim;
  unsigned long long* slots;
};

// gamma's sum in fixed point: the pass adds each fragment's fp64 partial, scaled by 2^(50 - e)
// where 2^e > the previous pack's total sum |w| (so the new total is about 2^50 units) and
// rounded to an integer, to one of kBandSlots counters. Integer sums do not depend on the order
// of the additions, so gamma is the same on every run; its rounding error (half a unit per
// fragment) is below 2^-33 of the total (1.2e-10), which the fix-up kernel checks (a total under
// frags * 2^32 units). A fragment above 2^62 / frags units (the total could overflow), or a previous
// sum of 0 or not finite, sets the overflow flag. In either case the fix-up kernel adds the fp64
// partials in a fixed order instead.
__device__ __forceinline__ double band_scale(float gamma_prev, double count) {
  const double tot = (double)gamma_prev * count;
  if (!(tot > 0.0) || !isfinite(tot)) return 0.0;
  int e;
  frexp(tot, &e);
  return ldexp(1.0, 50 - e);
}

// One workgroup per fragment. SINGLE = false: the second read of the two-pass pack (gamma_p is
// this pack's gamma; optional variance-correction counts and structured outliers). SINGLE =
// true: the single pass of a re-pack (gamma_p is the previous pack's gamma).
template <int M, int N, int FORM, bool SINGLE>
__global__ __launch_bounds__(256) void pack_lean(const float* __restrict__ w, int64_t ld_w,
                                                 int vec4, Layout L,
                                                 const float* __restrict__ gamma_p,
                                                 uint8_t* __restrict__ mask_plane,
                                                 uint8_t* __restrict__ code_plane,
                                                 uint32_t* __restrict__ flip_parts,
                                                 uint32_t* __restrict__ vc_parts,
                                                 const uint16_t* __restrict__ omask, BandWs band,
                                                 double count) {
  const int64_t frag = blockIdx.x;
  const int tid = threadIdx.x;
  const PieceAt p = piece_at<FORM>(L, frag, tid);
  uint16_t* mp = L.has_mask ? piece_mask<FORM>(mask_plane, frag, tid, p) : nullptr;
  const uint32_t old_keep = L.has_mask ? (uint32_t)*mp : 0u;
  uint32_t obits = 0u;
  if (!SINGLE && omask) {
    const int qpos = (int)(p.k0 - (frag % L.quads) * kQuadK);
    const int64_t oslot = (frag << 6) | ((p.lane_slot & 15) + 16 * (qpos >> 6));
    obits = omask[oslot * 4 + ((qpos & 63) >> 4)];
  }
  uint32_t u[16];
  load_piece(w, ld_w, vec4, p, u);
  if (!SINGLE && omask) {
#pragma unroll
    for (int i = 0; i < 16; ++i) u[i] = (obits >> i) & 1u ? 0u : u[i];
  }
  uint32_t a[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = u[i] & 0x7FFFFFFFu;
  const float half = 0.5f * gamma_p[0];
  const uint32_t hbits = __float_as_uint(half);
  uint32_t t_lo = hbits, t_hi = hbits;
  if constexpr (SINGLE) {
    t_lo = __float_as_uint(half * (1.0f - kBandHalfWidth));
    t_hi = __float_as_uint(half * (1.0f + kBandHalfWidth));
  }
  uint32_t v[16 / M];
  const uint32_t keep = lean_keep<M, N>(a, p.cnt, v);
  uint32_t cw;
  lean_codes<FORM>(u, a, keep, t_hi, &cw, p.word);
  reinterpret_cast<uint32_t*>(code_plane)[frag * 256 + tid] = cw;
  if (L.has_mask) {
    *mp = (uint16_t)keep;
    const uint32_t sum = wave_sum_u32((uint32_t)__builtin_popcount((old_keep ^ keep) & 0xFFFFu));
    if ((tid & 63) == 0) flip_parts[frag * 4 + (tid >> 6)] = sum;
  }
  if constexpr (!SINGLE) {
    if (vc_parts) {
      uint32_t nzd = 0;
#pragma unroll
      for (int i = 15; i >= 0; --i) nzd = shl_gt(nzd, a[i], hbits);
      const uint32_t d = wave_sum_u32((uint32_t)__builtin_popcount(nzd));
      const uint32_t sp = wave_sum_u32((uint32_t)__builtin_popcount(nzd & keep));
      if ((tid & 63) == 0) {
        vc_parts[(frag * 4 + (tid >> 6)) * 2] = d;
        vc_parts[(frag * 4 + (tid >> 6)) * 2 + 1] = sp;
      }
    }
  } else {
    // A kept magnitude inside (T_lo, T_hi]: kept ones are at or above their group's n-th
    // largest, so the test runs over [max(T_lo + 1, v), T_hi], as one unsigned compare of
    // 2a - 2 lo against 2 (T_hi - lo) (a value below lo wraps past it).
    // (One range for the thread's 16, from the smallest group threshold: a superset of the kept
    // ones. Positions past the row's end hold 0 and wrap, so they never count.)
    uint32_t lo = t_lo + 1u;
    if constexpr (N != M) {
      uint32_t vmin = v[0];
#pragma unroll
      for (int g = 1; g < 16 / M; ++g) vmin = min(vmin, v[g]);
      lo = max(lo, vmin);
    }
    const uint32_t c = 0u - 2u * lo;
    uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < 16; ++i) mn = min(mn, (u[i] << 1) + c);
    const bool inband = lo <= t_hi && mn <= 2u * (t_hi - lo);
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += (double)__uint_as_float(a[i]);
    s = wave_sum_f64(s);
    const uint64_t bal = __ballot(inband);
    __shared__ uint32_t wcount[4];
    __shared__ double wsum[4];
    const int wave = tid >> 6;
    if ((tid & 63) == 0) {
      wcount[wave] = (uint32_t)__popcll(bal);
      wsum[wave] = s;
    }
    __syncthreads();
    uint32_t base = 0;
#pragma unroll
    for (int i = 0; i < 3; ++i) base += i < wave ? wcount[i] : 0u;
    const uint32_t pos =
        base + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    uint8_t* const rec = band.seg + frag * kBandRecBytes;
    if (inband && pos < (uint32_t)kBandSegCap) rec[4 + pos] = (uint8_t)tid;
    if (tid == 0) {
      *reinterpret_cast<uint32_t*>(rec) = wcount[0] + wcount[1] + wcount[2] + wcount[3];
      const double part = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
      band.part[frag] = part;
      const double sc = band_scale(gamma_p[0], count);
      const double q = part * sc;
      if (sc > 0.0 && q < ldexp(1.0, 62) / (double)gridDim.x)
        atomicAdd(band.slots + 16 * (frag % kBandSlots), (unsigned long long)llrint(q));
      else
        atomicOr(band.lim + 2, 1u);
      if (frag == 0) {
        band.lim[0] = t_lo;
        band.lim[1] = t_hi;
        *reinterpret_cast<double*>(band.lim + 4) = sc;
      }
    }
  }
}

// The fix-up kernel of the single pass (after it in the stream). Every workgroup first adds the
// pass's per-fragment partial sums in one fixed order (thread t takes partials t, t + 1024, ...,
// then the waves' sums in wave order), so each computes the same gamma, and workgroup 0 stores it.
// With the new threshold H inside the pass's bracket, each listed piece re-reads its 16 weights
// and ORs in the nonzero codes of its kept magnitudes in (T_lo, T_hi] that exceed H (they were
// written as zero). A fragment that listed more pieces than its record holds, or every fragment
// when H left the bracket, has its code words rewritten from the weights and the stored keep
// bits. Workgroup b takes fragments b, b + G, ... (at most kFixFrags): their records and the
// partial sums are loaded together, then the listed pieces are spread over the threads.
constexpr int kFixFrags = 448;
template <int M, int N, int FORM>
__global__ __launch_bounds__(1024) void pack_fix(const float* __restrict__ w, int64_t ld_w,
                                                 int vec4, Layout L, float* __restrict__ gamma_out,
                                                 uint8_t* __restrict__ mask_plane,
                                                 uint8_t* __restrict__ code_plane, BandWs band,
                                                 int64_t frags, double count,
                                                 uint32_t* __restrict__ pack_gen) {
  constexpr int kWords = kBandRecBytes / 4;
  __shared__ uint32_t rec[kFixFrags][kWords];
  __shared__ uint32_t start[kFixFrags + 1];
  __shared__ uint32_t whole[kFixFrags];  // fragments rewritten whole (their k), nwhole of them
  __shared__ uint32_t wwhole[16];
  __shared__ uint32_t nwhole;
  __shared__ double wsum[16];
  __shared__ uint32_t wtot[16];
  __shared__ float gsh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t G = gridDim.x;
  const int nf = (int)min<int64_t>(kFixFrags, (frags - blockIdx.x + G - 1) / G);
  // records (16 bytes per load) and partial sums, loads in flight together
  constexpr int kRecVec = kBandRecBytes / 16;
#pragma unroll 4
  for (int j = tid; j < nf * kRecVec; j += 1024) {
    const int k = j / kRecVec, q = j % kRecVec;
    *reinterpret_cast<uint4*>(&rec[k][4 * q]) = reinterpret_cast<const uint4*>(
        band.seg + (blockIdx.x + (int64_t)k * G) * kBandRecBytes)[q];
  }
  // gamma: the fixed-point counters, or the fp64 partials if the pass flagged an overflow or the
  // counters' total is below frags * 2^32 units (the weights shrank by more than about 2^(17 -
  // log2 frags) since the previous pack: the half unit each fragment rounds off would then exceed
  // 2^-33 of the total)
  __shared__ bool use_fixed;
  if (tid == 0) use_fixed = false;
  __syncthreads();
  if (band.lim[2] == 0u && wave == 0) {
    const unsigned long long v = band.slots[16 * lane];
    // the 64 counters add up below 2^63
    unsigned long long sum = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) sum += __shfl_xor(sum, o, 64);
    if (lane == 0 && (double)sum >= (double)frags * 0x1p32) {
      const double sc = *reinterpret_cast<const double*>(band.lim + 4);  // the pass's scale
      gsh = count > 0.0 ? (float)(((double)sum / sc) / count) : 0.0f;
      use_fixed = true;
    }
  }
  __syncthreads();
  if (!use_fixed) {
    double acc = 0.0;
    for (int64_t i0 = 0; i0 < frags; i0 += 16 * 1024) {
      double v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int64_t i = i0 + tid + u * 1024;
        v[u] = i < frags ? band.part[i] : 0.0;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) acc += v[u];
    }
    acc = wave_sum_f64(acc);
    if (lane == 0) wsum[wave] = acc;
    __syncthreads();
    if (tid == 0) {
      double s = 0.0;
      for (int k = 0; k < 16; ++k) s += wsum[k];
      gsh = count > 0.0 ? (float)(s / count) : 0.0f;
    }
  }
  __syncthreads();
  if (tid == 0) {
    if (blockIdx.x == 0) {
      gamma_out[0] = gsh;
      pack_gen[0] += 1u;  // one more pack of the handle (the transposed plane is now stale)
    }
    // the last workgroup to have read the counters clears them for the next pass
    // Relaxed: a workgroup's counter loads have returned before its arrival (their sum is
    // computed above), and the clearing stores need only be visible to the next launch. (A
    // release here compiles to a write-back of the whole L2 per workgroup.)
    const uint32_t old = __hip_atomic_fetch_add(band.lim + 3, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    if (old == (uint32_t)G - 1) {
      for (int k = 0; k < kBandSlots; ++k) band.slots[16 * k] = 0ull;
      band.lim[2] = 0u;
      band.lim[3] = 0u;
    }
  }
  const uint32_t hbits = __float_as_uint(0.5f * gsh);
  const uint32_t t_lo = band.lim[0], t_hi = band.lim[1];
  const bool in_bracket = t_lo <= hbits && hbits <= t_hi;
  // listed pieces per fragment (0 for a fragment rewritten whole), exclusive prefix sums
  uint32_t c = 0;
  bool w_all = false;
  if (tid < nf) {
    const uint32_t r = rec[tid][0];
    w_all = !in_bracket || r > (uint32_t)kBandSegCap;
    c = w_all ? 0u : r;
  }
  // the fragments rewritten whole, listed in order
  {
    const uint64_t bal = __ballot(w_all);
    if (lane == 0) wwhole[wave] = (uint32_t)__popcll(bal);
    __syncthreads();
    uint32_t off = 0;
    for (int k = 0; k < wave; ++k) off += wwhole[k];
    if (w_all)
      whole[off + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                            __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] = tid;
    if (tid == 0) {
      uint32_t s = 0;
      for (int k = 0; k < 16; ++k) s += wwhole[k];
      nwhole = s;
    }
  }
  uint32_t x = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wtot[wave] = x;
  __syncthreads();
  uint32_t woff = 0;
  for (int k = 0; k < wave; ++k) woff += wtot[k];
  if (tid < nf) start[tid] = woff + x - c;
  if (tid == nf - 1) start[nf] = woff + x;
  __syncthreads();
  uint32_t* const words = reinterpret_cast<uint32_t*>(code_plane);
  const uint32_t total = start[nf];
  for (uint32_t e = tid; e < total; e += 1024) {
    int lo = 0, hi = nf - 1;  // the fragment k with start[k] <= e < start[k + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (start[mid] <= e) lo = mid; else hi = mid - 1;
    }
    const int k = lo;
    const int64_t frag = blockIdx.x + (int64_t)k * G;
    const int t = reinterpret_cast<const uint8_t*>(rec[k])[4 + (e - start[k])];
    const PieceAt p = piece_at<FORM>(L, frag, t);
    uint32_t u[16];
    load_piece(w, ld_w, vec4, p, u);
    const uint32_t keep =
        L.has_mask ? (uint32_t)*piece_mask<FORM>(mask_plane, frag, t, p) : 0xFFFFu;
    uint32_t orw = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t ai = u[i] & 0x7FFFFFFFu;
      if (!((keep >> i) & 1u) || ai <= t_lo || ai > t_hi || ai <= hbits) continue;
      const uint32_t neg = u[i] >> 31;
      if constexpr (FORM == kFormPositional) {
        orw |= (1u + neg) << (8 * (i & 3) + 2 * (i >> 2));
      } else {
        const int q = i >> 2;
        const uint32_t k4 = (keep >> (4 * q)) & 0xFu;
        const int hb = 31 - __builtin_clz(k4);
        const int slot = 8 * (p.word & 1) + 2 * q + ((i & 3) == hb ? 1 : 0);
        orw |= (1u << neg) << sp24_code_bit(slot);
      }
    }
    if (orw) atomicOr(words + frag * 256 + (FORM == kFormSparse24 ? (t & ~1) : t), orw);
  }
  // fragments rewritten whole: four at a time, 256 threads each
  const int sub = tid >> 8, st = tid & 255;
  const int nw = (int)nwhole;
  for (int j0 = 0; j0 < nw; j0 += 4) {
    const int j = j0 + sub;
    if (j >= nw) continue;  // uniform over each group of 256 threads
    const int64_t frag = blockIdx.x + (int64_t)whole[j] * G;
    const PieceAt p = piece_at<FORM>(L, frag, st);
    uint32_t u[16], a[16];
    load_piece(w, ld_w, vec4, p, u);
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = u[i] & 0x7FFFFFFFu;
    const uint32_t keep =
        L.has_mask ? (uint32_t)*piece_mask<FORM>(mask_plane, frag, st, p) : 0xFFFFu;
    uint32_t cw;
    lean_codes<FORM>(u, a, keep, hbits, &cw, p.word);
    words[frag * 256 + st] = cw;
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
// columns: its 512 bricks go to LDS as 2-bit codes in the positional word layout (16 positions
// per word; positional bricks are copied as they are, 2:4 slots are moved to their positions,
// kept-form bricks are decoded), every thread assembles 8 transposed words of 8 columns into an
// LDS copy of the workgroup's 16 output blocks, and the blocks (512 contiguous bytes each) are
// written with 16-byte stores. Rows past n_out are zero.
//
// LDS layouts, chosen so that no access has bank conflicts on gfx950's 64 four-byte banks:
//   code words: row r's 16 words start at 16 r + 16 (r >> 4), word c at c ^ 4 ((r >> 6) & 3).
//     The decode writes a row's 4 words of one brick with one 16-byte store (a wave covers 16
//     consecutive rows: 1 KB in 16 row segments); the assembly reads rows 32 g + 16 h + rr (fixed
//     rr) of 4 columns per wave, 32 distinct words that this layout puts in 32 distinct banks.
//   output blocks: word i of block cbl at 128 cbl + (i ^ 4 ((i >> 6) & 1) ^ 2 (cbl & 1)
//     ^ 8 ((cbl >> 1) & 1)). An assembly store (fixed column step) writes words 2 c + 32 g + h,
//     which would fold onto 16 banks; the block bits spread them over 64. The final read takes
//     each thread's 8 words as two 16-byte reads: the XORs keep 4-word groups whole (bit 1 only
//     swaps their halves, undone in registers), and bit 6 of i moved to bit 2 puts the 16 groups
//     of a quarter wave on 16 distinct 4-bank sets.
__device__ __forceinline__ int tc_cw_at(int r, int c) {
  return r * 16 + 16 * (r >> 4) + (c ^ (4 * ((r >> 6) & 3)));
}
__device__ __forceinline__ int tc_ow_at(int cbl, int i) {
  return cbl * 128 + (i ^ (((i >> 6) & 1) << 2) ^ ((cbl & 1) << 1) ^ (((cbl >> 1) & 1) << 3));
}

__global__ __launch_bounds__(256) void transpose_codes(Layout L, const uint8_t* mask_plane,
                                                       const uint8_t* code_plane,
                                                       int64_t rq_count,
                                                       uint32_t* __restrict__ tplane,
                                                       const uint32_t* __restrict__ pack_gen) {
  // Nothing to do when the plane was built from the handle's last pack (the data-gradient kernel
  // records that pack count once it has run on the plane).
  if (__builtin_amdgcn_readfirstlane((int)pack_gen[1]) ==
      __builtin_amdgcn_readfirstlane((int)pack_gen[0]))
    return;
  __shared__ __attribute__((aligned(16))) uint32_t cw[128 * 16 + 7 * 16];
  __shared__ __attribute__((aligned(16))) uint32_t ow[16 * 128];
  const int64_t rq = blockIdx.x / L.quads, q = blockIdx.x % L.quads;
  const int tid = threadIdx.x;
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i, rl = idx >> 2, b = idx & 3;
    const int64_t row = rq * 128 + rl;
    uint32_t w4[4] = {0u, 0u, 0u, 0u};
    if (row < L.n_out) {
      const int64_t brick = q * kFragBricks + b;
      if (L.form == kFormSparse24) {
        // the brick's 64 positions are lane groups 2 (b & 1) + hh of block b >> 1 of the quad:
        // slot j of a lane group's code word (bits 8 (j & 3) + 2 (j >> 2)) goes to position
        // 4 (j >> 1) + index_j of its 32, i.e. word j >> 3, bits 8 index_j + 2 ((j >> 1) & 3)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int64_t s2 =
              (((row >> 4) * L.quads + q) << 6) | ((row & 15) + 16 * (2 * (b & 1) + hh));
          const uint2 ci = *reinterpret_cast<const uint2*>(code_plane + s2 * 16 + 8 * (b >> 1));
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const uint32_t c = (ci.x >> sp24_code_bit(j)) & 3u, p = (ci.y >> (2 * j)) & 3u;
            w4[2 * hh + (j >> 3)] |= c << (8 * p + 2 * ((j >> 1) & 3));
          }
        }
      } else if (L.positional) {
        // already 2-bit codes in the layout below
        const uint4 v =
            *reinterpret_cast<const uint4*>(code_plane + brick_slot(L, row, brick) * 16);
        w4[0] = v.x;
        w4[1] = v.y;
        w4[2] = v.z;
        w4[3] = v.w;
      } else {
        uint32_t mask[2], dec[16];
        decode_brick(L, mask_plane, code_plane, row, brick, mask, dec);
        for (int j = 0; j < kBrickK; ++j) {
          const uint32_t v = (dec[j >> 2] >> (8 * (j & 3))) & 0xFFu;
          w4[j >> 4] |= (v == 0xFFu ? 2u : v) << pos_bit(j & 15);
        }
      }
    }
    *reinterpret_cast<uint4*>(&cw[tc_cw_at(rl, 4 * b)]) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  }
  __syncthreads();
  const int task = tid >> 1, half = tid & 1;
  const int cbl = task >> 3, g = (task >> 1) & 3, h = task & 1;
  uint32_t rw[16];
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) rw[rr] = cw[tc_cw_at(32 * g + 16 * h + rr, cbl)];
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) {
    // column c = 8 half + cc of the word's 16 sits at bits 8 (c & 3) + 2 (c >> 2)
    const int sh = 8 * (cc & 3) + 4 * half + 2 * (cc >> 2);
    uint32_t out = 0;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)  // rr = 8 s + 2 p + e
      out |= ((rw[rr] >> sh) & 3u) << (2 * ((rr >> 1) & 3) + 8 * (rr >> 3) + 16 * (rr & 1));
    ow[tc_ow_at(cbl, (8 * half + cc + 16 * g) * 2 + h)] = out;
  }
  __syncthreads();
  // 16 threads per output block, 8 consecutive words (32 bytes) each
  const int ob = tid >> 4, part = tid & 15;
  uint4* const dst = reinterpret_cast<uint4*>(tplane + ((q * 16 + ob) * rq_count + rq) * 128 +
                                              8 * part);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint4 v = *reinterpret_cast<const uint4*>(&ow[tc_ow_at(ob, 8 * part + 4 * k) & ~3]);
    dst[k] = (ob & 1) ? make_uint4(v.z, v.w, v.x, v.y) : v;
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

// Lean kernels of a pattern and form: calls FN(M, N, FORM) for the template arguments, or
// returns false when the pattern has none (the kept form, and patterns outside the lean set).
template <typename Fn>
bool with_lean(const Layout& L, Fn&& fn) {
  if (L.form == kFormKept || !lean_pattern(L.n, L.m)) return false;
  if (L.form == kFormSparse24) {
    fn(std::integral_constant<int, 4>{}, std::integral_constant<int, 2>{},
       std::integral_constant<int, kFormSparse24>{});
  } else if (L.n == L.m) {
    fn(std::integral_constant<int, 16>{}, std::integral_constant<int, 16>{},
       std::integral_constant<int, kFormPositional>{});
  } else if (L.m == 4) {
    fn(std::integral_constant<int, 4>{}, std::integral_constant<int, 2>{},
       std::integral_constant<int, kFormPositional>{});
  } else if (L.m == 8 && L.n == 4) {
    fn(std::integral_constant<int, 8>{}, std::integral_constant<int, 4>{},
       std::integral_constant<int, kFormPositional>{});
  } else if (L.m == 8) {
    fn(std::integral_constant<int, 8>{}, std::integral_constant<int, 6>{},
       std::integral_constant<int, kFormPositional>{});
  } else {
    fn(std::integral_constant<int, 16>{}, std::integral_constant<int, 8>{},
       std::integral_constant<int, kFormPositional>{});
  }
  return true;
}

hipError_t launch_pack(const float* w, int64_t ld_w, sbn_packed* h, hipStream_t s) {
  const Layout& L = h->L;
  const int vec4 = ((uintptr_t)w % 16 == 0) && (ld_w % 4 == 0) && (L.K % 4 == 0);
  const bool outl = h->outlier_k > 0 && L.n_out > 0;
  const int64_t frags = L.row_blocks_pad * L.quads;
  const BandWs band{h->band_part, h->band_seg, h->band_lim, h->band_slots};
  // A re-pack without outliers or variance correction reads the latent weights once.
  const bool single = h->gamma_valid && h->band_part != nullptr && !outl && !h->vc &&
                      L.n_out > 0 && L.form != kFormKept && lean_pattern(L.n, L.m);
  h->single_pass = single;
  if (single) {
    with_lean(L, [&](auto MM, auto NN, auto FF) {
      hipLaunchKernelGGL((pack_lean<decltype(MM)::value, decltype(NN)::value, decltype(FF)::value, true>), dim3((unsigned)frags), dim3(256), 0,
                         s, w, ld_w, vec4, L, h->gamma, h->mask, h->codes, h->flip_parts,
                         nullptr, nullptr, band, (double)L.n_out * (double)L.K);
      // 128 workgroups (fewer for few fragments), more if one would take over kFixFrags; on the
      // 7B re-packs 32, 64, 128 and 256 measured 13.3, 10.9, 10.2 and 17 us at 2:4
      const int64_t fix_blocks = std::max<int64_t>(std::min<int64_t>(128, (frags + 3) / 4),
                                                   (frags + kFixFrags - 1) / kFixFrags);
      hipLaunchKernelGGL((pack_fix<decltype(MM)::value, decltype(NN)::value, decltype(FF)::value>),
                         dim3((unsigned)fix_blocks), dim3(1024), 0, s, w, ld_w, vec4, L, h->gamma,
                         h->mask, h->codes, band, frags, (double)L.n_out * (double)L.K,
                         h->pack_gen);
    });
  } else {
    if (L.n_out > 0) {
      hipLaunchKernelGGL(absmean_partial, dim3(h->num_partials), dim3(kAbsmeanThreads), 0, s, w,
                         L.n_out, L.K, ld_w, vec4, h->partials);
    }
    if (outl) {
      hipError_t e = launch_outlier_select(w, ld_w, h, s);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(absmean_finalize, dim3(1), dim3(kAbsmeanThreads), 0, s, h->partials,
                       L.n_out > 0 ? h->num_partials : 0, (double)L.n_out * (double)L.K, h->gamma,
                       outl ? h->osum : nullptr,
                       outl ? (L.n_out * (L.K >> 8) + 255) / 256 : (int64_t)0, h->pack_gen);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || L.n_out == 0) return e;
    uint32_t* const vc = h->vc ? h->vc_parts : nullptr;
    const uint16_t* const om = outl ? reinterpret_cast<const uint16_t*>(h->omask) : nullptr;
    const bool lean = with_lean(L, [&](auto MM, auto NN, auto FF) {
      hipLaunchKernelGGL((pack_lean<decltype(MM)::value, decltype(NN)::value, decltype(FF)::value, false>), dim3((unsigned)frags), dim3(256), 0,
                         s, w, ld_w, vec4, L, h->gamma, h->mask, h->codes, h->flip_parts, vc, om,
                         band, 0.0);
    });
    if (!lean) {
      const dim3 grid((unsigned)frags);
#define SBN_PACK(MM, FF)                                                                      \
  hipLaunchKernelGGL((pack_fragments<MM, FF>), grid, dim3(256), 0, s, w, ld_w, vec4, L, h->gamma, \
                     h->mask, h->codes, h->flip_parts, vc, om)
      if (L.m == 4) {
        if (L.positional) SBN_PACK(4, kFormPositional); else SBN_PACK(4, kFormKept);
      } else if (L.m == 8) {
        if (L.positional) SBN_PACK(8, kFormPositional); else SBN_PACK(8, kFormKept);
      } else {
        if (L.positional) SBN_PACK(16, kFormPositional); else SBN_PACK(16, kFormKept);
      }
#undef SBN_PACK
    }
  }
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
                     h->mask, h->codes, h->rq_count, h->tplane, h->pack_gen);
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
