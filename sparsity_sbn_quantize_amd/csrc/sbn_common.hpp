// Shared device-side definitions of the packed ternary weight layout.
//
// Packed format (per output row, per group of m consecutive weights along K; Sparse-BitNet,
// Abstract and Figure 6 for the n-of-m selection; "bitnet.cpp: Matrix-Free Inference" for the
// four-per-byte 2-bit codes): the n kept codes of a group, in ascending position, as 2-bit two's
// complement (00 = 0, 01 = +1, 11 = -1), LSB first; and, when n < m, an m-bit keep mask (bit i <->
// position i of the group).
//
// Kernel layout ("brick fragments"). A brick is 64 consecutive K positions of one row: its mask
// bits (64 bits = 8 bytes, absent when n == m) and its code bits (64/m groups * 2n bits =
// 16n/m bytes). Because every brick holds whole groups, a row's code and mask streams are the
// concatenation of its bricks' bits, so the per-row reference bitstreams are recovered by
// copying bricks. Bricks are stored fragment-major: 16 rows x 4 bricks (one 16x16x64 MFMA
// A-operand tile over 256 K) form 64 bricks stored contiguously in lane order
// (lane = row % 16 + 16 * (brick % 4)), so that one wave-wide load of one brick per lane reads
// one contiguous block. Rows are padded to a multiple of 16 and bricks to a multiple of 4 with
// zero bricks (all pruned, code 0); for the benchmarked shapes no padding occurs. The mask plane
// and the code plane are separate arrays.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sbn {

constexpr int kBrickK = 64;         // K positions per brick
constexpr int kFragRows = 16;       // rows per fragment
constexpr int kFragBricks = 4;      // bricks per fragment (along K)
constexpr int kQuadK = kBrickK * kFragBricks;  // 256 K positions per fragment

struct Layout {
  int64_t n_out, K;
  int n, m;
  int code_brick_bytes;  // 16 n / m
  int has_mask;          // n < m
  int64_t row_blocks;    // ceil(n_out / 16)
  int64_t quads;         // ceil(ceil(K / 64) / 4)
};

__host__ __device__ inline int64_t brick_slot(const Layout& L, int64_t row, int64_t brick) {
  const int64_t rb = row >> 4, bq = brick >> 2;
  const int64_t lane = (row & 15) | ((brick & 3) << 4);
  return ((rb * L.quads + bq) << 6) | lane;
}

// 2-bit two's complement code -> int8 byte (10 is never written; it decodes as 0).
__host__ __device__ constexpr uint32_t code_to_byte(uint32_t c) {
  return c == 1u ? 0x01u : (c == 3u ? 0xFFu : 0x00u);
}

// Order of the code bits inside a brick. A brick holding S codes (S = 64n/m, in group order, each
// group's kept codes in ascending position) stores them either in plain order (code i at bits
// [2i, 2i+2) of the brick's code words, as in the per-row bitstream) or, when S % 16 == 0, in
// plane order: code 16w + 4q + i at bits [8i + 2q, 8i + 2q + 2) of code word w. In plane order
// the four codes 16w+4q .. 16w+4q+3 are the bytes of (word >> 2q) & 0x03030303, so sixteen codes
// become int8 bytes with three ALU ops per four codes and no table.
__host__ __device__ constexpr bool plane_order(int n, int m) { return (64 * n / m) % 16 == 0; }

__host__ __device__ constexpr int code_bit(int i, bool plane) {
  return plane ? (i >> 4) * 32 + 8 * (i & 3) + 2 * ((i >> 2) & 3) : 2 * i;
}

// Sixteen 2-bit codes: sequence order (code c at bits 2c) <-> plane order (code 4q+i at 8i+2q).
__host__ __device__ inline uint32_t seq_to_plane(uint32_t s) {
  uint32_t p = 0;
  for (int c = 0; c < 16; ++c) p |= ((s >> (2 * c)) & 3u) << (8 * (c & 3) + 2 * (c >> 2));
  return p;
}
__host__ __device__ inline uint32_t plane_to_seq(uint32_t p) {
  uint32_t s = 0;
  for (int c = 0; c < 16; ++c) s |= ((p >> (8 * (c & 3) + 2 * (c >> 2))) & 3u) << (2 * c);
  return s;
}

// Selector table of one mask byte (8 positions): byte p = rank of position p among the kept
// positions below it when bit p is set, else 12 (v_perm's constant-zero selector).
__host__ __device__ constexpr uint64_t sel8_entry(uint32_t m8) {
  uint64_t v = 0;
  uint32_t rank = 0;
  for (int p = 0; p < 8; ++p) {
    uint64_t b = 12;
    if ((m8 >> p) & 1u) b = rank++;
    v |= b << (8 * p);
  }
  return v;
}

// Plain (table-free) decode of one brick into 16 dwords of int8 weights: dword p holds
// positions 4p..4p+3. Works for any n:m; used by export and the generic forward path.
__device__ inline void decode_brick_plain(const uint32_t mask[2], const uint32_t codes[4], int n,
                                          int m, int has_mask, uint32_t out[16]) {
  const bool plane = plane_order(n, m);
  const int groups = kBrickK / m;
  int idx = 0;  // running code index in the brick
#pragma unroll 1
  for (int g = 0; g < groups; ++g) {
#pragma unroll 1
    for (int i = 0; i < m; ++i) {
      const int pos = g * m + i;
      uint32_t kept = has_mask ? ((mask[pos >> 5] >> (pos & 31)) & 1u) : 1u;
      uint32_t b = 0;
      if (kept) {
        const int bit = code_bit(idx, plane);  // 2-bit fields never straddle a word
        b = code_to_byte((codes[bit >> 5] >> (bit & 31)) & 3u);
        ++idx;
      }
      const int d = pos >> 2, s = (pos & 3) * 8;
      out[d] = (out[d] & ~(0xFFu << s)) | (b << s);
    }
  }
}

// Sixteen codes of a plane-order code word -> four words of int8 bytes (sequence order).
__device__ __forceinline__ void conv16(uint32_t w, uint32_t* out) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    out[q] = __builtin_amdgcn_perm(0u, 0xFF000100u, (w >> (2 * q)) & 0x03030303u);
}

// Table decode of one brick for the patterns with a fast path (n:m in {2:4, 4:8, 6:8, 8:16} and
// the dense n == m). `sel` points at this lane's replica of the selector table in LDS:
// sel[m8 * 16] is the entry of mask byte m8. Codes are in plane order.
template <int N, int M>
__device__ __forceinline__ void decode_brick_sel(const uint2* __restrict__ sel,
                                                 const uint32_t mask[2], const uint32_t codes[4],
                                                 uint32_t out[16]) {
  constexpr int kCodes = kBrickK * N / M;  // codes in the brick
  uint32_t cv[kCodes / 4];                 // codes as int8 bytes, sequence order
#pragma unroll
  for (int w = 0; w < kCodes / 16; ++w) conv16(codes[w], cv + 4 * w);
  if constexpr (N == M) {
#pragma unroll
    for (int d = 0; d < 16; ++d) out[d] = cv[d];
  } else if constexpr (M == 4 || (M == 8 && N == 4)) {
    // Every 8 positions hold exactly 4 kept codes: conv word h.
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const uint32_t m8 = (mask[h >> 2] >> (8 * (h & 3))) & 0xFFu;
      const uint2 s = sel[m8 * 16];
      out[2 * h] = __builtin_amdgcn_perm(0u, cv[h], s.x);
      out[2 * h + 1] = __builtin_amdgcn_perm(0u, cv[h], s.y);
    }
  } else if constexpr (M == 8 && N == 6) {
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const uint32_t m8 = (mask[g >> 2] >> (8 * (g & 3))) & 0xFFu;
      const uint2 s = sel[m8 * 16];
      const int k = (6 * g) >> 2;
      uint32_t lo, hi;
      if ((g & 1) == 0) {
        lo = cv[k];
        hi = cv[k + 1];
      } else {  // the group's codes start at byte 2 of cv[k]
        lo = __builtin_amdgcn_alignbyte(cv[k + 1], cv[k], 2);
        hi = cv[k + 1] >> 16;
      }
      out[2 * g] = __builtin_amdgcn_perm(hi, lo, s.x);
      out[2 * g + 1] = __builtin_amdgcn_perm(hi, lo, s.y);
    }
  } else if constexpr (M == 16 && N == 8) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t m16 = (mask[g >> 1] >> (16 * (g & 1))) & 0xFFFFu;
      const uint32_t lo8 = m16 & 0xFFu, hi8 = m16 >> 8;
      const uint2 sl = sel[lo8 * 16];
      const uint2 sh = sel[hi8 * 16];
      const uint32_t c0 = cv[2 * g], c1 = cv[2 * g + 1];
      out[4 * g] = __builtin_amdgcn_perm(c1, c0, sl.x);
      out[4 * g + 1] = __builtin_amdgcn_perm(c1, c0, sl.y);
      // The upper half's codes follow the popcount(lo8) codes of the lower half.
      const uint64_t win = ((((uint64_t)c1 << 32) | c0) >> ((8 * __builtin_popcount(lo8)) & 63));
      out[4 * g + 2] = __builtin_amdgcn_perm((uint32_t)(win >> 32), (uint32_t)win, sh.x);
      out[4 * g + 3] = __builtin_amdgcn_perm((uint32_t)(win >> 32), (uint32_t)win, sh.y);
    }
  }
}

// Decodes K-slice j (positions 16j..16j+15, the A operand of MFMA j) of one brick for the fast
// patterns; same arithmetic as decode_brick_sel, restricted to one slice so that a caller can
// overwrite slice j of its A registers as soon as MFMA j has consumed them.
template <int N, int M>
__device__ __forceinline__ void decode_slice_sel(const uint2* __restrict__ sel,
                                                 const uint32_t mask[2], const uint32_t codes[4],
                                                 int j, uint32_t out[4]) {
  auto conv = [&](int k) -> uint32_t {  // codes [4k, 4k+4) of the brick as int8 bytes
    return __builtin_amdgcn_perm(0u, 0xFF000100u, (codes[k >> 2] >> (2 * (k & 3))) & 0x03030303u);
  };
  if constexpr (N == M) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = conv(4 * j + i);
  } else if constexpr (M == 4 || (M == 8 && N == 4)) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int h = 2 * j + hh;
      const uint32_t m8 = (mask[h >> 2] >> (8 * (h & 3))) & 0xFFu;
      const uint2 s = sel[m8 * 16];
      const uint32_t c = conv(h);
      out[2 * hh] = __builtin_amdgcn_perm(0u, c, s.x);
      out[2 * hh + 1] = __builtin_amdgcn_perm(0u, c, s.y);
    }
  } else if constexpr (M == 8 && N == 6) {
    const uint32_t c0 = conv(3 * j), c1 = conv(3 * j + 1), c2 = conv(3 * j + 2);
    const int g0 = 2 * j, g1 = 2 * j + 1;
    const uint2 s0 = sel[((mask[g0 >> 2] >> (8 * (g0 & 3))) & 0xFFu) * 16];
    const uint2 s1 = sel[((mask[g1 >> 2] >> (8 * (g1 & 3))) & 0xFFu) * 16];
    out[0] = __builtin_amdgcn_perm(c1, c0, s0.x);
    out[1] = __builtin_amdgcn_perm(c1, c0, s0.y);
    const uint32_t lo = __builtin_amdgcn_alignbyte(c2, c1, 2), hi = c2 >> 16;
    out[2] = __builtin_amdgcn_perm(hi, lo, s1.x);
    out[3] = __builtin_amdgcn_perm(hi, lo, s1.y);
  } else if constexpr (M == 16 && N == 8) {
    const uint32_t c0 = conv(2 * j), c1 = conv(2 * j + 1);
    const uint32_t m16 = (mask[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    const uint32_t lo8 = m16 & 0xFFu, hi8 = m16 >> 8;
    const uint2 sl = sel[lo8 * 16];
    const uint2 sh = sel[hi8 * 16];
    out[0] = __builtin_amdgcn_perm(c1, c0, sl.x);
    out[1] = __builtin_amdgcn_perm(c1, c0, sl.y);
    const uint64_t win = ((((uint64_t)c1 << 32) | c0) >> ((8 * __builtin_popcount(lo8)) & 63));
    out[2] = __builtin_amdgcn_perm((uint32_t)(win >> 32), (uint32_t)win, sh.x);
    out[3] = __builtin_amdgcn_perm((uint32_t)(win >> 32), (uint32_t)win, sh.y);
  }
}

// Patterns decoded by decode_brick_sel.
__host__ __device__ constexpr bool sel_fast_path(int n, int m) {
  return n == m || (m == 4 && n == 2) || (m == 8 && (n == 4 || n == 6)) || (m == 16 && n == 8);
}

// Fills the replicated selector table: 256 entries x 16 replicas of 8 bytes (32 KB), replica r
// of entry e at sel[e * 16 + r]. Each lane reads its own replica (lane % 16), so the 16 lanes
// that an LDS cycle serves for 8-byte reads never share a bank.
__device__ __forceinline__ void fill_sel_table(uint2* sel) {
  for (int e = threadIdx.x; e < 256; e += blockDim.x) {
    const uint64_t v = sel8_entry((uint32_t)e);
    const uint2 w = make_uint2((uint32_t)v, (uint32_t)(v >> 32));
#pragma unroll
    for (int r = 0; r < 16; ++r) sel[e * 16 + ((r + e) & 15)] = w;  // rotate to spread banks
  }
}

}  // namespace sbn
