// Structured outliers ("From 2:4 to 8:16 sparsity patterns in LLMs for Outliers and Weights with
// Variance Correction", summary: salient weights are kept in structured 4:256, 8:256 or 16:256
// patterns, about 1.5, 3.1 and 6.25 percent of the weights).
//
// In each group of 256 consecutive weights along K, the k of largest |w| (equal magnitudes: the
// lower position first) are kept apart as bf16 values. The ternary n:m path sees the other weights
// only: their positions read as 0 for the absmean scale, the keep mask and the codes. The forward
// adds their term to the fp32 output:
//
//   y[t][r] = fl32( y_ternary[t][r] + fl32( o[t][r] * fl32(a'_t / 127) ) )
//   o[t][r] = sum over the row's outliers of x_q[t][position] * value   (fp32; every product of an
//             int8 and a bf16 value is exact; the additions run in a fixed order)
//
// Planes (allocated with the handle when K % 256 == 0, for k up to 16):
//   opos  [G][k][n_out] uint8   positions within the group, ascending for each row and group
//   oval  [G][k][n_out] uint16  bf16 bit patterns (round to nearest even of the latent fp32)
//   omask brick layout of the mask plane (one 64-bit word per brick slot): the outlier positions
//   osum  [ceil(n_out G / 256)]  fp64 sum of the outlier |w| of each selection workgroup (a fixed
//                               order), subtracted from the absmean sum
// (G = K / 256; entry (g, j) of all rows is contiguous, so the forward's loads coalesce.)
#include "sbn_internal.hpp"

namespace sbn {
namespace {

// One thread per (row, group). Every weight becomes a key (|w| bits, then 256 - position: larger
// keys rank first, equal magnitudes rank the lower position first) and passes through a chain of
// KO compare-and-swap steps that keeps the KO largest keys in order. The positions are then sorted
// ascending and written out with their values and mask bits; the workgroup's outlier |w| sum goes
// to osum[blockIdx.x].
template <int KO>
__global__ __launch_bounds__(256) void outlier_select(const float* __restrict__ w, int64_t ld_w,
                                                      int vec4, Layout L,
                                                      uint8_t* __restrict__ opos,
                                                      uint16_t* __restrict__ oval,
                                                      unsigned long long* __restrict__ omask,
                                                      double* __restrict__ osum) {
  __shared__ double red[4];
  const int64_t G = L.K >> 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = idx < L.n_out * G;
  const int64_t r = live ? idx / G : 0, g = live ? idx % G : 0;
  const float* wr = w + r * ld_w + g * 256;
  unsigned long long key[KO];
#pragma unroll
  for (int i = 0; i < KO; ++i) key[i] = 0ull;  // below every real key
  auto insert = [&](float v, int p) {
    unsigned long long kk =
        ((unsigned long long)(__float_as_uint(v) & 0x7FFFFFFFu) << 9) | (unsigned)(256 - p);
#pragma unroll
    for (int i = 0; i < KO; ++i) {
      const unsigned long long t = key[i];
      const bool gt = kk > t;
      key[i] = gt ? kk : t;
      kk = gt ? t : kk;
    }
  };
#pragma unroll 2
  for (int p = 0; p < 256; p += 4) {
    if (vec4) {
      const float4 f = *reinterpret_cast<const float4*>(wr + p);
      insert(f.x, p);
      insert(f.y, p + 1);
      insert(f.z, p + 2);
      insert(f.w, p + 3);
    } else {
      for (int u = 0; u < 4; ++u) insert(wr[p + u], p + u);
    }
  }
  int pos[KO];
#pragma unroll
  for (int i = 0; i < KO; ++i) pos[i] = 256 - (int)(key[i] & 511ull);
#pragma unroll
  for (int i = 1; i < KO; ++i) {  // insertion sort, ascending
#pragma unroll
    for (int j = i; j > 0; --j) {
      const int a = pos[j - 1], b = pos[j];
      pos[j - 1] = min(a, b);
      pos[j] = max(a, b);
    }
  }
  unsigned long long bm[4] = {0ull, 0ull, 0ull, 0ull};
  double s = 0.0;
  if (live) {
#pragma unroll
    for (int j = 0; j < KO; ++j) {
      const int p = pos[j];
      const float v = wr[p];
      const int64_t o = (g * KO + j) * L.n_out + r;
      opos[o] = (uint8_t)p;
      oval[o] = (uint16_t)bf16_rne(v);
      bm[p >> 6] |= 1ull << (p & 63);
      s += (double)fabsf(v);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) omask[brick_slot(L, r, g * 4 + b)] = bm[b];
  }
  // workgroup sum in a fixed order: wave sums (DPP tree), then the four waves in order
  s = wave_sum_f64(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) osum[blockIdx.x] = ((red[0] + red[1]) + red[2]) + red[3];
}

// Outlier term of the forward: a workgroup takes 256 / C rows and a tile of TT tokens, whose int8
// activations it stages in LDS. Thread (c, row) walks groups c, c + C, ... of its row (the next
// group's positions and values are loaded while the current one is used) and sums the products
// for its TT tokens; with C > 1 (few tokens: more threads per row) the C partial sums of a row
// meet in LDS in the order c = 0, 1, ... . The row's sum o then goes into y as fl32(o * step).
template <int KO, int TT, int C>
__global__ __launch_bounds__(256) void outlier_add(Layout L, const uint8_t* __restrict__ opos,
                                                   const uint16_t* __restrict__ oval,
                                                   const int8_t* __restrict__ xq, int64_t ld_q,
                                                   const float* __restrict__ absmax, int64_t T,
                                                   float* __restrict__ y, int64_t ld_y) {
  extern __shared__ int8_t xs[];  // [TT][K]
  constexpr int kRows = 256 / C;
  __shared__ float part[C > 1 ? C : 1][kRows][TT];
  const int c = threadIdx.x / kRows, rl = threadIdx.x % kRows;
  const int64_t r = (int64_t)blockIdx.x * kRows + rl;
  const int64_t t0 = (int64_t)blockIdx.y * TT;
  const int nt = (int)min<int64_t>(TT, T - t0);
  const int K = (int)L.K;
  const bool v16 = ((uintptr_t)xq % 16 == 0) && (ld_q % 16 == 0);  // K % 256 == 0 here
  for (int tt = 0; tt < nt; ++tt) {
    const int8_t* src = xq + (t0 + tt) * ld_q;
    if (v16) {
      for (int k = 16 * threadIdx.x; k < K; k += 16 * 256)
        *reinterpret_cast<uint4*>(xs + tt * K + k) = *reinterpret_cast<const uint4*>(src + k);
    } else {
      for (int k = threadIdx.x; k < K; k += 256) xs[tt * K + k] = src[k];
    }
  }
  __syncthreads();
  float o[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) o[tt] = 0.0f;
  const int64_t G = L.K >> 8;
  if (r < L.n_out && c < G) {
    uint32_t pk[KO], vk[KO];
    auto load = [&](int64_t g) {
#pragma unroll
      for (int j = 0; j < KO; ++j) {
        const int64_t e = (g * KO + j) * L.n_out + r;
        pk[j] = opos[e];
        vk[j] = oval[e];
      }
    };
    load(c);
    for (int64_t g = c; g < G; g += C) {
      uint32_t p[KO];
      float v[KO];
#pragma unroll
      for (int j = 0; j < KO; ++j) {
        p[j] = (uint32_t)(g * 256) + pk[j];
        v[j] = __uint_as_float(vk[j] << 16);
      }
      if (g + C < G) load(g + C);
#pragma unroll
      for (int j = 0; j < KO; ++j) {  // position order within the group
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          if (tt < nt) o[tt] = __fadd_rn(o[tt], __fmul_rn((float)xs[tt * K + p[j]], v[j]));
        }
      }
    }
  }
  if constexpr (C > 1) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) part[c][rl][tt] = o[tt];
    __syncthreads();
    if (c != 0) return;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      float sum = part[0][rl][tt];
#pragma unroll
      for (int cc = 1; cc < C; ++cc) sum = __fadd_rn(sum, part[cc][rl][tt]);
      o[tt] = sum;
    }
  }
  if (r >= L.n_out) return;
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    if (tt < nt) {
      const float step = absmax[t0 + tt] / 127.0f;
      float* dst = y + (t0 + tt) * ld_y + r;
      *dst = __fadd_rn(*dst, __fmul_rn(o[tt], step));
    }
  }
}

// Export: per row, the group's k positions and bf16 values in [n_out][G][k] order.
__global__ __launch_bounds__(256) void export_outliers(Layout L, int KO, const uint8_t* opos,
                                                       const uint16_t* oval, uint8_t* pos_out,
                                                       uint16_t* val_out) {
  const int64_t G = L.K >> 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (g, j, r), r fastest
  if (idx >= G * KO * L.n_out) return;  // (g, j) entries of all rows
  const int64_t r = idx % L.n_out, gj = idx / L.n_out;
  const int64_t dst = r * G * KO + gj;
  if (pos_out) pos_out[dst] = opos[idx];
  if (val_out) val_out[dst] = oval[idx];
}

}  // namespace

hipError_t launch_outlier_select(const float* w, int64_t ld_w, const sbn_packed* h,
                                 hipStream_t s) {
  const Layout& L = h->L;
  const int64_t groups = L.n_out * (L.K >> 8);
  if (groups == 0) return hipSuccess;
  const int vec4 = ((uintptr_t)w % 16 == 0) && (ld_w % 4 == 0);
  const dim3 grid((unsigned)((groups + 255) / 256));
  if (h->outlier_k == 4) {
    hipLaunchKernelGGL(outlier_select<4>, grid, dim3(256), 0, s, w, ld_w, vec4, L, h->opos,
                       h->oval, h->omask, h->osum);
  } else if (h->outlier_k == 8) {
    hipLaunchKernelGGL(outlier_select<8>, grid, dim3(256), 0, s, w, ld_w, vec4, L, h->opos,
                       h->oval, h->omask, h->osum);
  } else {
    hipLaunchKernelGGL(outlier_select<16>, grid, dim3(256), 0, s, w, ld_w, vec4, L, h->opos,
                       h->oval, h->omask, h->osum);
  }
  return hipGetLastError();
}

hipError_t launch_outlier_add(const sbn_packed* h, const int8_t* xq, int64_t ld_q,
                              const float* absmax, int64_t T, float* y, int64_t ld_y,
                              hipStream_t s) {
  const Layout& L = h->L;
  if (T == 0 || L.n_out == 0) return hipSuccess;
  // token tile: 1 for one token, else 4 or 16 as T and 64 KB of staged activations allow
  const int tt = T == 1 ? 1 : ((T > 4 && 16 * L.K <= 65536) ? 16 : (4 * L.K <= 65536 ? 4 : 1));
  const size_t smem = (size_t)tt * (size_t)L.K;
  // few tokens: 8 threads per row (32 rows per workgroup); a token tile of 16: one per row
#define SBN_OUTL(KK, TTV)                                                                      \
  do {                                                                                         \
    constexpr int CC = TTV == 16 ? 1 : 8;                                                      \
    hipError_t e = allow_smem(outlier_add<KK, TTV, CC>, smem);                                 \
    if (e != hipSuccess) return e;                                                             \
    const dim3 grid((unsigned)((L.n_out + 256 / CC - 1) / (256 / CC)),                         \
                    (unsigned)((T + tt - 1) / tt));                                            \
    hipLaunchKernelGGL((outlier_add<KK, TTV, CC>), grid, dim3(256), smem, s, L, h->opos,       \
                       h->oval, xq, ld_q, absmax, T, y, ld_y);                                 \
  } while (0)
#define SBN_OUTL_T(KK)                                                                         \
  do {                                                                                         \
    if (tt == 1) SBN_OUTL(KK, 1); else if (tt == 4) SBN_OUTL(KK, 4); else SBN_OUTL(KK, 16);    \
  } while (0)
  if (h->outlier_k == 4) SBN_OUTL_T(4);
  else if (h->outlier_k == 8) SBN_OUTL_T(8);
  else SBN_OUTL_T(16);
#undef SBN_OUTL_T
#undef SBN_OUTL
  return hipGetLastError();
}

hipError_t launch_export_outliers(const sbn_packed* h, uint8_t* pos, uint16_t* val,
                                  hipStream_t s) {
  const Layout& L = h->L;
  const int64_t total = (L.K >> 8) * h->outlier_k * L.n_out;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(export_outliers, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, L,
                     h->outlier_k, h->opos, h->oval, pos, val);
  return hipGetLastError();
}

}  // namespace sbn
