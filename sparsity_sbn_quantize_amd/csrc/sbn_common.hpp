// Shared device-side definitions of the packed ternary weight layout.
//
// What a packed weight holds (Sparse-BitNet, Abstract and Figure 6 for the n-of-m selection;
// "bitnet.cpp: Matrix-Free Inference" for 2-bit ternary codes, four per byte): per output row and
// per group of m consecutive weights along K, an m-bit keep mask (bit i <-> position i of the
// group; absent when n == m) and the ternary codes of the kept positions.
//
// Kernel layout ("brick fragments"). A brick is 64 consecutive K positions of one row: its mask
// bits (8 bytes, absent when n == m) and its code bits. Bricks are stored fragment-major: 16 rows
// x 4 bricks (one 16x16x64 MFMA A-operand tile over 256 K) form 64 bricks stored contiguously in
// lane order (lane = row % 16 + 16 * (brick % 4)), so that one wave-wide load of one brick per lane
// reads one contiguous block. Rows are padded to a multiple of 256 and bricks to a multiple of 4
// with zero bricks (all pruned, code 0). The mask plane and the code plane are separate arrays.
//
// Codes come in one of three forms:
//   - positional (2n >= m: 2:4, 4:8, 6:8, 8:16 and dense n == m). Every position of the brick has
//     a 2-bit code, 0 where pruned: 16 bytes per brick, as many bits per weight as the reference
//     format's kept codes plus mask when n == m/2 and fewer when n > m/2 (e.g. 2 vs 2.5 bits for
//     6:8). The forward reads only this plane. Position p is at bits [8i + 2q, 8i + 2q + 2) of
//     code word w, where p = 16w + 4q + i, with 00 = 0, 01 = +1, 10 = -1; so the sixteen
//     positions of word w become int8 bytes with nine ALU ops (exp_word_to_i8).
//   - sparse 2:4 (the operands of gfx950's structured-sparse MFMA v_smfmac_i32_16x16x128_i8):
//     per lane (row r = lane % 16, lane group g = lane / 16) and 256-K quad, four words: for each
//     128-K block b, a code word with the 16 kept codes of K [128b + 32g, 128b + 32g + 32) (slot j
//     = the lower (j even) or higher (j odd) kept position of group j / 2 of 4; slot 4q + i at bits
//     8i + 2q, positional values), then an index word (slot j's position in its group at bits
//     [2j, 2j + 2)). 16 bytes per lane per quad, the same as positional codes.
//   - kept (2n < m): the n kept codes of each group in ascending position, 2-bit two's complement
//     (00 = 0, 01 = +1, 11 = -1), code i of the brick at bits [2i, 2i+2): exactly the reference
//     bitstream, 16n/m bytes per brick. Decoded with decode_kept_brick.
//
// Compact plane (inference only; written next to the planes above when a pack asks for it and
// read by the GEMV). A product needs only which positions are nonzero and their signs, so per
// brick it holds a 64-bit nonzero mask (bit i <-> position i) and csb = 64n/m sign bits: group g
// of the brick owns slots [g*n, g*n + n), slot g*n + j is 1 when the group's j-th nonzero code in
// ascending position is -1, and unused slots are 0. A fragment quad stores its 64 lanes' masks (8
// bytes each, lane order) and then the lanes' sign bits as one bit stream (lane l at stream bits
// [l*csb, (l+1)*csb), little-endian words): 512 + 8*csb bytes per quad, (m + n)/m bits per weight
// (1.5 at 2:4 and 8:16, 1.75 at 6:8).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sbn {

constexpr int kBrickK = 64;         // K positions per brick
constexpr int kFragRows = 16;       // rows per fragment
constexpr int kFragBricks = 4;      // bricks per fragment (along K)
constexpr int kQuadK = kBrickK * kFragBricks;  // 256 K positions per fragment

enum CodeForm : int {
  kFormPositional = 0,
  kFormKept = 1,
  kFormSparse24 = 2,
  // compact plane, by group size (kernel template forms only; Layout::form never holds these)
  kFormCompact4 = 3,
  kFormCompact8 = 4,
  kFormCompact16 = 5
};

__host__ __device__ constexpr bool compact_form(int f) { return f >= kFormCompact4; }
__host__ __device__ constexpr int compact_m(int f) {
  return f == kFormCompact4 ? 4 : (f == kFormCompact8 ? 8 : 16);
}
constexpr int kCompactMaskBytes = 64 * 8;  // nonzero masks of one fragment quad
constexpr int kCompactSlack = 16;          // zero bytes after the plane (3-word sign loads)
__host__ __device__ constexpr int64_t compact_quad_bytes(int csb) {
  return kCompactMaskBytes + 8 * (int64_t)csb;
}

struct Layout {
  int64_t n_out, K;
  int n, m;
  int form;              // CodeForm
  int positional;        // form != kFormKept: 16 code bytes per lane and quad
  int code_brick_bytes;  // 16, or 16 n / m for the kept form
  int has_mask;          // n < m
  int64_t row_blocks;    // ceil(n_out / 16)
  int64_t row_blocks_pad;  // row_blocks rounded up to kPadRowBlocks (stored, zero-filled)
  int64_t quads;         // ceil(ceil(K / 64) / 4)
  int csb;               // compact plane: sign bits per brick, 64 n / m
};

// Stored row fragments are padded with zero bricks to a multiple of 16 (256 rows), so that a GEMM
// tile never addresses past the planes.
constexpr int kPadRowBlocks = 16;

__host__ __device__ constexpr bool positional_codes(int n, int m) { return 2 * n >= m; }

// Sparse 2:4 form: dense positions (0..31 of the lane's 32) of the 16 slots of a code/index pair.
__device__ __forceinline__ int sp24_pos(uint32_t index_word, int j) {
  return 4 * (j >> 1) + (int)((index_word >> (2 * j)) & 3u);
}
// Slot j's code bits inside a code word (slot 4q + i at bits 8i + 2q).
__host__ __device__ constexpr int sp24_code_bit(int j) { return 8 * (j & 3) + 2 * (j >> 2); }

__host__ __device__ inline int64_t brick_slot(const Layout& L, int64_t row, int64_t brick) {
  const int64_t rb = row >> 4, bq = brick >> 2;
  const int64_t lane = (row & 15) | ((brick & 3) << 4);
  return ((rb * L.quads + bq) << 6) | lane;
}

// Bit offset of brick position p (0..63) in the positional code words.
__host__ __device__ constexpr int pos_bit(int p) {
  return (p >> 4) * 32 + 8 * (p & 3) + 2 * ((p >> 2) & 3);
}

// Positional 2-bit code of a ternary value and back.
__host__ __device__ constexpr uint32_t pos_code(int v) { return v > 0 ? 1u : (v < 0 ? 2u : 0u); }
__host__ __device__ constexpr int pos_value(uint32_t c) { return c == 1u ? 1 : (c == 2u ? -1 : 0); }

// Reference (two's complement) 2-bit code of a ternary value and back (10 is never written).
__host__ __device__ constexpr uint32_t ref_code(int v) { return v > 0 ? 1u : (v < 0 ? 3u : 0u); }
__host__ __device__ constexpr int ref_value(uint32_t c) { return c == 1u ? 1 : (c == 3u ? -1 : 0); }

// One positional code word (positions 16w .. 16w+15) -> four words of int8 bytes, word q holding
// positions 16w + 4q .. 16w + 4q + 3. Each output word is one v_perm whose selector bytes are the
// masked codes: for q even the codes sit in bits 0-1 of each byte (selector 0, 1, 2 picks byte
// 0x00, 0x01, 0xFF of 0x00FF0100); for q odd in bits 2-3 (selector 0 picks 0x00 of the second
// source, 4 picks 0x01 of the first, 8 replicates the sign bit of byte 1 of 0x00008000, 0xFF).
__device__ __forceinline__ void exp_word_to_i8(uint32_t w, uint32_t out[4]) {
  const uint32_t w4 = w >> 4;
  out[0] = __builtin_amdgcn_perm(0u, 0x00FF0100u, w & 0x03030303u);
  out[1] = __builtin_amdgcn_perm(1u, 0x00008000u, w & 0x0C0C0C0Cu);
  out[2] = __builtin_amdgcn_perm(0u, 0x00FF0100u, w4 & 0x03030303u);
  out[3] = __builtin_amdgcn_perm(1u, 0x00008000u, w4 & 0x0C0C0C0Cu);
}

// Half h of exp_word_to_i8: its output words 2h and 2h + 1 (for spreading a decode over the MFMA
// groups it overlaps).
__device__ __forceinline__ void exp_word_half_to_i8(uint32_t w, int h, uint32_t& o0, uint32_t& o1) {
  const uint32_t v = h ? w >> 4 : w;
  o0 = __builtin_amdgcn_perm(0u, 0x00FF0100u, v & 0x03030303u);
  o1 = __builtin_amdgcn_perm(1u, 0x00008000u, v & 0x0C0C0C0Cu);
}

// Plain decode of one kept-form brick into 16 dwords of int8 weights: dword p holds positions
// 4p..4p+3. Works for any n:m; used by export and by the forward for the kept form.
__device__ inline void decode_kept_brick(const uint32_t mask[2], const uint32_t codes[4], int n,
                                         int m, int has_mask, uint32_t out[16]) {
  (void)n;
  const int groups = kBrickK / m;
  int idx = 0;  // running code index in the brick
#pragma unroll 1
  for (int g = 0; g < groups; ++g) {
#pragma unroll 1
    for (int i = 0; i < m; ++i) {
      const int pos = g * m + i;
      const uint32_t kept = has_mask ? ((mask[pos >> 5] >> (pos & 31)) & 1u) : 1u;
      uint32_t b = 0;
      if (kept) {
        const int bit = 2 * idx;  // 2-bit fields never straddle a word
        b = (uint32_t)ref_value((codes[bit >> 5] >> (bit & 31)) & 3u) & 0xFFu;
        ++idx;
      }
      const int d = pos >> 2, s = (pos & 3) * 8;
      out[d] = (out[d] & ~(0xFFu << s)) | (b << s);
    }
  }
}

// Compact nibble table: entry m4 | s << 4 holds the int8 codes of four positions whose nonzero
// bits are m4, the nonzero ones taking their signs from the low bits of s in order (1 = -1).
__host__ __device__ inline uint32_t compact_nibble_entry(uint32_t e) {
  const uint32_t m4 = e & 15u, s = e >> 4;
  uint32_t out = 0, k = 0;
  for (int i = 0; i < 4; ++i) {
    if ((m4 >> i) & 1u) {
      out |= (((s >> k) & 1u) ? 0xFFu : 0x01u) << (8 * i);
      ++k;
    }
  }
  return out;
}

// Decodes one compact brick into 16 words of int8 codes (word d = positions 4d .. 4d+3).
// mask: the brick's nonzero mask; sg_lo, sg_hi: its sign slots 0..63; n, csb: the pattern's n and
// 64 n / m; lut: the 256-entry nibble table. Half h of the brick (positions 32h .. 32h+31) holds
// whole groups whose slots are [h csb/2, (h+1) csb/2), at most 32 bits, so each half reads one
// 32-bit window. Nibble j starts at slot off = its group's first slot plus the nonzero positions
// before it in the group; off never passes the window's end except for a nibble with no nonzero
// position (its group's slots are used up), whose table row is all zero for any s.
template <int M>
__device__ __forceinline__ void decode_compact(const uint32_t mask[2], uint32_t sg_lo,
                                               uint32_t sg_hi, int n, int csb,
                                               const uint32_t* lut, uint32_t out[16]) {
  const int half_bits = csb >> 1;
  const uint32_t w1 =
      half_bits >= 32 ? sg_hi : __builtin_amdgcn_alignbit(sg_hi, sg_lo, (uint32_t)half_bits);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t mw = mask[h], sw = h ? w1 : sg_lo;
    uint32_t off = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j % (M / 4) == 0) off = (uint32_t)((4 * j / M) * n);
      const uint32_t m4 = (mw >> (4 * j)) & 15u;
      const uint32_t s4 = __builtin_amdgcn_ubfe(sw, off, 4u);
      out[8 * h + j] = lut[m4 | (s4 << 4)];
      off += (uint32_t)__builtin_popcount(m4);
    }
  }
}

// Per-token absmax INT8 quantization helpers, shared by the quantize kernel and the fused decode
// forward so that both produce identical bytes:
//   a' = max(max |x|, 1e-5); s = fl32(127 / a'); q = clamp(rne(fl32(x * s)), -127, 127).
constexpr float kAbsmaxFloor = 1e-5f;

// Running maximum of bf16 magnitudes, two per word (the sign cleared, 15-bit patterns compare
// in the order of the values for finite inputs).
__device__ __forceinline__ uint32_t max_abs_bf16x2(uint32_t acc, uint32_t w) {
  const uint32_t a = w & 0x7FFF7FFFu;
  const uint32_t lo = max(acc & 0xFFFFu, a & 0xFFFFu);
  const uint32_t hi = max(acc >> 16, a >> 16);
  return lo | (hi << 16);
}

// Four bf16 (two per word) -> four int8 packed in a word.
__device__ __forceinline__ uint32_t quant4(uint32_t w01, uint32_t w23, float s) {
  const float f0 = __uint_as_float(w01 << 16), f1 = __uint_as_float(w01 & 0xFFFF0000u);
  const float f2 = __uint_as_float(w23 << 16), f3 = __uint_as_float(w23 & 0xFFFF0000u);
  const int i0 = (int)__builtin_amdgcn_fmed3f(__builtin_rintf(f0 * s), -127.f, 127.f);
  const int i1 = (int)__builtin_amdgcn_fmed3f(__builtin_rintf(f1 * s), -127.f, 127.f);
  const int i2 = (int)__builtin_amdgcn_fmed3f(__builtin_rintf(f2 * s), -127.f, 127.f);
  const int i3 = (int)__builtin_amdgcn_fmed3f(__builtin_rintf(f3 * s), -127.f, 127.f);
  return (uint32_t)(i0 & 0xFF) | ((uint32_t)(i1 & 0xFF) << 8) | ((uint32_t)(i2 & 0xFF) << 16) |
         ((uint32_t)(i3 & 0xFF) << 24);
}

// Maximum over the 64 lanes of a wave of two packed 16-bit magnitudes (as max_abs_bf16x2), with
// DPP lane moves (no LDS round trips): within quads (xor 1, 2), half rows and rows (mirrors), then
// across rows (row broadcasts); lane 63 ends with the result, which is returned to every lane.
__device__ __forceinline__ uint32_t wave_max_u16x2(uint32_t v) {
  auto dpp = [](uint32_t old, uint32_t x, int ctrl, int row_mask) -> uint32_t {
    switch (ctrl) {  // the control word must be a constant expression
      case 0xB1: return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, 0xB1, 0xF, 0xF, false);
      case 0x4E: return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, 0x4E, 0xF, 0xF, false);
      case 0x141: return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, 0x141, 0xF, 0xF, false);
      case 0x140: return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, 0x140, 0xF, 0xF, false);
      case 0x142: return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, 0x142, 0xA, 0xF, false);
      default: return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, 0x143, 0xC, 0xF, false);
    }
    (void)row_mask;
  };
  v = max_abs_bf16x2(v, dpp(v, v, 0xB1, 0xF));   // quad_perm [1,0,3,2]
  v = max_abs_bf16x2(v, dpp(v, v, 0x4E, 0xF));   // quad_perm [2,3,0,1]
  v = max_abs_bf16x2(v, dpp(v, v, 0x141, 0xF));  // row_half_mirror
  v = max_abs_bf16x2(v, dpp(v, v, 0x140, 0xF));  // row_mirror
  v = max_abs_bf16x2(v, dpp(v, v, 0x142, 0xA));  // row_bcast:15 into rows 1, 3
  v = max_abs_bf16x2(v, dpp(v, v, 0x143, 0xC));  // row_bcast:31 into rows 2, 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Sum over the 64 lanes of a wave with the same DPP lane moves as wave_max_u16x2. The row
// broadcasts write only rows 1, 3 (then 2, 3); the other rows add 0.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);  // row_mirror
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// GEMM tile order. Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2).
// The linear block id is remapped so that every XCD receives one contiguous run of tiles in a
// grouped order (kTileGroup token tiles x all N tiles, N-major within the group): the tiles an
// XCD has in flight then share activation rows and packed weights in its L2.
constexpr int kXcds = 8;
constexpr int kTileGroup = 4;

// Position of block `bid` in the XCD-contiguous order.
__device__ __forceinline__ int xcd_order(int nblocks, int bid) {
  const int xcd = bid % kXcds, j = bid / kXcds;
  const int base = nblocks / kXcds, extra = nblocks % kXcds;
  return xcd * base + min(xcd, extra) + j;
}

// Tile of position `lin` in the grouped order.
__device__ __forceinline__ void grouped_tile(int lin, int tiles_n, int tiles_t, int& tile_n,
                                             int& tile_t) {
  const int per_group = kTileGroup * tiles_n;
  const int group = lin / per_group, r = lin % per_group;
  const int gsize = min(kTileGroup, tiles_t - group * kTileGroup);
  tile_n = r / gsize;
  tile_t = group * kTileGroup + r % gsize;
}

// One DPP lane move of a double (both halves); lanes of rows outside RMASK read 0.0.
template <int CTRL, int RMASK>
__device__ __forceinline__ double dpp_f64(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, RMASK, 0xF,
                                                            false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL,
                                                            RMASK, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Sum over the 64 lanes of a wave in fp64 (the lane moves of wave_sum_u32); every lane gets the
// value of lane 63.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_f64<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_f64<0x140, 0xF>(v);  // row_mirror
  v += dpp_f64<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_f64<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Combining one value per wave of a workgroup (at most 16 waves): lane w holds wave w's value
// (0 for lanes past the last wave), and four DPP steps inside the first row of 16 lanes (two quad
// permutations, then the half-row and row mirrors) leave the result in every lane of that row;
// lane 0's copy is returned. One LDS read and a few ALU steps, instead of a read per wave.
__device__ __forceinline__ uint32_t row16_max_u16x2(uint32_t v) {
  v = max_abs_bf16x2(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
  v = max_abs_bf16x2(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
  v = max_abs_bf16x2(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));
  v = max_abs_bf16x2(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
}
__device__ __forceinline__ double row16_sum_f64(double v) {
  v += dpp_f64<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_f64<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_f64<0x140, 0xF>(v);  // row_mirror
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 0);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 0);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Round an fp32 value to a bf16 bit pattern, nearest even (finite values).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Parameter-free LayerNorm of two bf16 values (one word) with fp32 mean mu and 1/sigma r:
// bf16(fl32(fl32(x - mu) * r)) each.
__device__ __forceinline__ uint32_t ln_pair(uint32_t w, float mu, float r) {
  const float z0 = __fmul_rn(__fsub_rn(__uint_as_float(w << 16), mu), r);
  const float z1 = __fmul_rn(__fsub_rn(__uint_as_float(w & 0xFFFF0000u), mu), r);
  return bf16_rne(z0) | (bf16_rne(z1) << 16);
}

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v3u __attribute__((ext_vector_type(3)));
typedef __attribute__((address_space(3))) void* lds_ptr;

// Word 3 of a raw buffer resource on gfx9 (32-bit data format, no swizzle, no stride): offsets are
// bytes and reads at or past num_records return zero.
constexpr int kBufDword3 = 0x00020000;

// s_waitcnt immediate that waits until at most `n` vector-memory operations are outstanding and
// does not wait on LDS/scalar or export counters (gfx9 encoding: vmcnt split over bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_imm(int n) {
  return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14);
}

}  // namespace sbn
