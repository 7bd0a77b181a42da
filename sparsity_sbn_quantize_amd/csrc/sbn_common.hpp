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

// Nibble expansion table: index (mask nibble << 8) | (next 8 code bits). Entry: the four int8
// weights of the nibble's positions, byte p = position p. Positions whose mask bit is clear are
// 0; set bits consume the next 2-bit code in order.
struct NibbleTable {
  uint32_t v[4096];
};

constexpr NibbleTable make_nibble_table() {
  NibbleTable t{};
  for (uint32_t mn = 0; mn < 16; ++mn) {
    for (uint32_t cb = 0; cb < 256; ++cb) {
      uint32_t word = 0, j = 0;
      for (uint32_t p = 0; p < 4; ++p) {
        if ((mn >> p) & 1u) {
          word |= code_to_byte((cb >> (2 * j)) & 3u) << (8 * p);
          ++j;
        }
      }
      t.v[(mn << 8) | cb] = word;
    }
  }
  return t;
}

// Plain (table-free) decode of one brick into 16 dwords of int8 weights: dword p holds
// positions 4p..4p+3. Works for any n:m; used by export and the generic forward path.
__device__ inline void decode_brick_plain(const uint32_t mask[2], const uint32_t codes[4], int n,
                                          int m, int has_mask, uint32_t out[16]) {
  const int groups = kBrickK / m;
  int bit = 0;  // running position in the code stream
#pragma unroll 1
  for (int g = 0; g < groups; ++g) {
#pragma unroll 1
    for (int i = 0; i < m; ++i) {
      const int pos = g * m + i;
      uint32_t kept = has_mask ? ((mask[pos >> 5] >> (pos & 31)) & 1u) : 1u;
      uint32_t b = 0;
      if (kept) {
        const uint32_t c = (codes[bit >> 5] >> (bit & 31)) & 3u;  // 2-bit fields never straddle
        b = code_to_byte(c);
        bit += 2;
      }
      const int d = pos >> 2, s = (pos & 3) * 8;
      out[d] = (out[d] & ~(0xFFu << s)) | (b << s);
    }
  }
}

// Table decode of one brick for a compile-time pattern N:M. `lut` is the nibble table in LDS.
template <int N, int M>
__device__ __forceinline__ void decode_brick_lut(const uint32_t* __restrict__ lut,
                                                 const uint32_t mask[2], const uint32_t codes[4],
                                                 uint32_t out[16]) {
  constexpr int kGroups = kBrickK / M;
  constexpr int kGroupCodeBits = 2 * N;
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    // The group's code bits, at a compile-time offset in the brick's code words.
    const int start = g * kGroupCodeBits;
    const int w = start >> 5, s = start & 31;
    uint32_t gw;
    if (s == 0) {
      gw = codes[w];
    } else if (s + kGroupCodeBits <= 32) {
      gw = codes[w] >> s;
    } else {
      gw = __builtin_amdgcn_alignbit(codes[w + 1], codes[w], s);
    }
    if constexpr (kGroupCodeBits < 32) gw &= (1u << kGroupCodeBits) - 1u;
    if constexpr (N == M) {
      // Dense: every position kept; nibble q of the group uses code bits [8q, 8q+8).
#pragma unroll
      for (int q = 0; q < M / 4; ++q) {
        const uint32_t cb = (gw >> (8 * q)) & 0xFFu;
        out[(g * M) / 4 + q] = lut[0xF00u | cb];
      }
    } else {
      uint32_t off = 0;  // kept codes consumed so far in this group
#pragma unroll
      for (int q = 0; q < M / 4; ++q) {
        const int pos = g * M + 4 * q;
        const uint32_t mn = (mask[pos >> 5] >> (pos & 31)) & 0xFu;
        const uint32_t cb = q == 0 ? (gw & 0xFFu) : __builtin_amdgcn_ubfe(gw, 2 * off, 8);
        out[pos >> 2] = lut[(mn << 8) | cb];
        if (q + 1 < M / 4) off += __builtin_popcount(mn);
      }
    }
  }
}

}  // namespace sbn
