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
// Each lane decodes one brick (64 K positions of one weight row) straight into the A operand of
// v_mfma_i32_16x16x64_i8: the brick's K slice j (positions 16j .. 16j+15) feeds MFMA j of the
// 256-K fragment. The B operand (activations) uses the same K assignment, so the products pair
// correctly whatever the instruction's internal K order. With positional codes one slice is one
// code word and becomes int8 bytes with nine ALU ops; the kept form (2n < m) is expanded with a
// plain loop over its mask.
//
//   GEMV (T <= 16): one workgroup per one or two 16-row fragment rows, its 4 waves split K; the
//   activations are staged once in LDS.
//   GEMM (T > 16): a workgroup computes 256 rows x 128 tokens; the 128 x 256 activation tile of
//   each K step is staged in LDS and shared by the waves.
#include "sbn_internal.hpp"

namespace sbn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i mfma16(const uint32_t* a, v4i b, v4i c) {
  const v4i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3]};
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b, c, 0, 0, 0);
}

// Loads one brick: positional codes (16 bytes), or the kept form's mask (8 bytes) and code bytes.
template <bool POS>
__device__ __forceinline__ void load_brick(const Layout& L, const uint8_t* __restrict__ mask_plane,
                                           const uint8_t* __restrict__ code_plane, int64_t slot,
                                           uint32_t mask[2], uint32_t codes[4]) {
  mask[0] = mask[1] = 0;
  codes[0] = codes[1] = codes[2] = codes[3] = 0;
  if constexpr (POS) {
    const uint4 c = *reinterpret_cast<const uint4*>(code_plane + slot * 16);
    codes[0] = c.x; codes[1] = c.y; codes[2] = c.z; codes[3] = c.w;
  } else {
    if (L.has_mask) {
      const uint2 m = *reinterpret_cast<const uint2*>(mask_plane + slot * 8);
      mask[0] = m.x;
      mask[1] = m.y;
    }
    const int cbb = L.code_brick_bytes;
    const uint8_t* c = code_plane + slot * cbb;
    for (int i = 0; i < cbb; ++i) codes[i >> 2] |= (uint32_t)c[i] << (8 * (i & 3));
  }
}

template <bool POS>
__device__ __forceinline__ void decode(const Layout& L, const uint32_t mask[2],
                                       const uint32_t codes[4], uint32_t out[16]) {
  if constexpr (POS) {
#pragma unroll
    for (int j = 0; j < 4; ++j) exp_word_to_i8(codes[j], out + 4 * j);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) out[i] = 0;
    decode_kept_brick(mask, codes, L.n, L.m, L.has_mask, out);
  }
}

// 16 activation bytes of one token row at K offset k (a multiple of 16), zero beyond K.
// XVEC: rows are 16-byte aligned and K % 16 == 0, so a chunk is either whole or absent.
template <bool XVEC>
__device__ __forceinline__ v4i load_x16(const int8_t* __restrict__ row, int k, int K) {
  if constexpr (XVEC) {
    // Branch-free: the load address is clamped into the row (K >= 16 here), the value masked.
    const v4i v = *reinterpret_cast<const v4i*>(row + min(k, K - 16));
    return k < K ? v : v4i{0, 0, 0, 0};
  } else {
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll 1
    for (int i = 0; i < 16; ++i) {
      if (k + i < K) w[i >> 2] |= (uint32_t)(uint8_t)row[k + i] << (8 * (i & 3));
    }
    return v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
  }
}

// 16 activation bytes at K offset k (a multiple of 16) with the address clamped into the row:
// bytes at k >= K are arbitrary row data, which is harmless wherever the weights at those
// positions are zero (bricks are zero-padded past K). XVEC rows only. No value select, so the
// load's result is not needed until it is used (no wait right after the load).
__device__ __forceinline__ v4i load_x16_clamped(const int8_t* __restrict__ row, int k, int K) {
  return *reinterpret_cast<const v4i*>(row + min(k, K - 16));
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

// GEMV (T <= 16): a workgroup owns RB 16-row fragment rows; its 4 waves split K (wave w takes
// the 256-K steps w, w+4, ...). K is walked in chunks of 16 steps (4096 K): the chunk's bricks
// are loaded first, then the chunk's activations are staged once in LDS (shared by all waves and
// row fragments instead of being re-read from L2 by every wave), then bricks are decoded and
// multiplied. Partial sums of the 4 waves are combined through LDS.
constexpr int kGemvChunk = 4;                       // K steps per wave per chunk
constexpr int kGemvChunkK = 4 * kGemvChunk * kQuadK;  // 4096
constexpr int kGemvXStride = kGemvChunkK + 16;

template <bool POS, bool XVEC, int RB>
__global__ __launch_bounds__(256) void bitlinear_gemv(
    const uint8_t* __restrict__ mask_plane, const uint8_t* __restrict__ code_plane, Layout L,
    const float* __restrict__ gamma_p, const int8_t* __restrict__ xq, int64_t ld_q,
    const float* __restrict__ absmax, int64_t T, void* __restrict__ y, int64_t ld_y,
    int out_kind) {
  __shared__ v4i red[3][RB][64];
  extern __shared__ __attribute__((aligned(16))) int8_t xs[];  // [T][kGemvXStride]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t rb0 = (int64_t)blockIdx.x * RB;
  const int t = lane & 15, g = lane >> 4;
  const int Ti = (int)T;
  const bool tok_ok = t < Ti;
  v4i acc[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) acc[r] = v4i{0, 0, 0, 0};
  uint32_t mask[kGemvChunk][RB][2], codes[kGemvChunk][RB][4];

  const int nchunks = (int)((L.quads + 4 * kGemvChunk - 1) / (4 * kGemvChunk));
  for (int c = 0; c < nchunks; ++c) {
    const int64_t qbase = (int64_t)c * 4 * kGemvChunk;
#pragma unroll
    for (int i = 0; i < kGemvChunk; ++i) {
      const int64_t q = qbase + wave + 4 * i;
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if (q < L.quads && rb0 + r < L.row_blocks) {
          load_brick<POS>(L, mask_plane, code_plane, (((rb0 + r) * L.quads + q) << 6) | lane,
                          mask[i][r], codes[i][r]);
        } else {
          mask[i][r][0] = mask[i][r][1] = 0;
          codes[i][r][0] = codes[i][r][1] = codes[i][r][2] = codes[i][r][3] = 0;
        }
      }
    }
    // Stage this chunk's activations: T rows x 4096 K in 16-byte pieces.
    const int k0 = c * kGemvChunkK;
    if (c > 0) __syncthreads();  // previous chunk's readers are done with xs
    for (int e = threadIdx.x; e < Ti * (kGemvChunkK / 16); e += 256) {
      const int tok = e / (kGemvChunkK / 16), ch = e % (kGemvChunkK / 16);
      *reinterpret_cast<v4i*>(xs + tok * kGemvXStride + ch * 16) =
          load_x16<XVEC>(xq + tok * ld_q, k0 + ch * 16, (int)L.K);
    }
    __syncthreads();
    const int8_t* xb = xs + (tok_ok ? t : 0) * kGemvXStride + g * kBrickK;
#pragma unroll
    for (int i = 0; i < kGemvChunk; ++i) {
      const int64_t q = qbase + wave + 4 * i;
      if (q < L.quads) {
        v4i b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          b[j] = tok_ok ? *reinterpret_cast<const v4i*>(xb + (wave + 4 * i) * kQuadK + 16 * j)
                        : v4i{0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          uint32_t a[16];
          decode<POS>(L, mask[i][r], codes[i][r], a);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[r] = mfma16(a + 4 * j, b[j], acc[r]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RB; ++r)
    if (wave > 0) red[wave - 1][r][lane] = acc[r];
  __syncthreads();
  if (wave != 0 || !tok_ok) return;
  const float gamma = gamma_p[0];
  const float step = out_kind == SBN_OUT_F32 ? absmax[t] / 127.0f : 0.0f;
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const v4i sum = acc[r] + red[0][r][lane] + red[1][r][lane] + red[2][r][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = (rb0 + r) * 16 + 4 * g + i;
      if (row < L.n_out) store_out(y, ld_y, out_kind, t, row, sum[i], gamma, step);
    }
  }
}

// GEMM: a workgroup of 8 waves computes 256 rows x (16*CF) tokens; wave w owns 2 row fragments
// (32 rows) and all tokens.
// K advances 256 per step. Activation tiles go global -> LDS directly (global_load_lds, no
// registers) into a 3-buffer ring, two steps ahead; each token row's 16-byte chunks are stored
// XOR-swizzled (chunk c at position c ^ (token % 16)) so that the fragment reads of 16 tokens
// hit distinct banks. Bricks of the next step are decoded K-slice by K-slice into the A
// registers right after the MFMAs that last read that slice, and the scheduler is asked to
// interleave that decode with the MFMAs. One barrier per step.
constexpr int kGemmWaves = 8;   // waves per workgroup: two per SIMD, so that one wave's decode
                                // and LDS traffic overlap the other's MFMAs
constexpr int kRF = 2;          // 16-row fragments per wave (256 rows per workgroup)
constexpr int kGemmCF = 8;      // 16-token fragments per workgroup (128 tokens)
constexpr int kXBufs = 3;       // activation ring depth
constexpr int kGemmThreads = kGemmWaves * 64;

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2). The linear block
// id is remapped so that every XCD receives one contiguous run of tiles in a grouped order
// (kTileGroup token tiles x all N tiles, N-major within the group): the tiles an XCD has in
// flight then share activation rows and packed weights in its L2.
constexpr int kXcds = 8;
constexpr int kTileGroup = 4;

__device__ __forceinline__ void xcd_tile(int nblocks, int bid, int tiles_n, int tiles_t,
                                         int& tile_n, int& tile_t) {
  const int xcd = bid % kXcds, j = bid / kXcds;
  const int base = nblocks / kXcds, extra = nblocks % kXcds;
  const int lin = xcd * base + min(xcd, extra) + j;  // position in the grouped order
  const int per_group = kTileGroup * tiles_n;
  const int group = lin / per_group, r = lin % per_group;
  const int gsize = min(kTileGroup, tiles_t - group * kTileGroup);
  tile_n = r / gsize;
  tile_t = group * kTileGroup + r % gsize;
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// s_waitcnt immediate that waits until at most `n` vector-memory operations are outstanding and
// does not wait on LDS/scalar or export counters (gfx9 encoding: vmcnt split over bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }

template <bool POS, int CF, bool XVEC>
__global__ __launch_bounds__(kGemmThreads, 1) void bitlinear_gemm(
    const uint8_t* __restrict__ mask_plane, const uint8_t* __restrict__ code_plane, Layout L,
    const float* __restrict__ gamma_p, const int8_t* __restrict__ xq, int64_t ld_q,
    const float* __restrict__ absmax, int64_t T, void* __restrict__ y, int64_t ld_y,
    int out_kind, int tiles_n, int tiles_t) {
  constexpr int kTok = CF * 16;
  constexpr int kTileBytes = kTok * kQuadK;  // one step's activation tile (no padding)
  constexpr int kXLoads = kTok * 16 / kGemmThreads;  // 16-byte pieces per thread per step
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int8_t* xs0 = reinterpret_cast<int8_t*>(smem);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int tile_n, tile_t;
  xcd_tile((int)gridDim.x, (int)blockIdx.x, tiles_n, tiles_t, tile_n, tile_t);
  const int64_t rb0 = ((int64_t)tile_n * kGemmWaves + wave) * kRF;
  const int64_t t0 = (int64_t)tile_t * kTok;
  const int64_t nq = L.quads;
  const int K = (int)L.K;
  const bool has_mask = !POS && L.has_mask != 0;
  const int cbb = POS ? 16 : L.code_brick_bytes;  // code bytes per brick

  // Brick addresses (rows past n_out are clamped: valid reads, results never stored).
  const uint8_t* mrow[kRF];
  const uint8_t* crow[kRF];
#pragma unroll
  for (int rf = 0; rf < kRF; ++rf) {
    const int64_t rb = min(rb0 + rf, L.row_blocks - 1);
    mrow[rf] = mask_plane + ((rb * nq) << 6 | lane) * 8;
    crow[rf] = code_plane + ((rb * nq) << 6 | lane) * cbb;
  }
  // This thread's activation pieces: wave-instruction i covers 4 tokens (lane / 16) x 16 chunk
  // positions (lane % 16); position p of token `tok` holds global chunk p ^ (tok % 16). Tokens
  // past T are clamped (never stored).
  const int8_t* xrow[kXLoads];
  int xchunk[kXLoads];
#pragma unroll
  for (int i = 0; i < kXLoads; ++i) {
    const int tok = 4 * (wave * kXLoads + i) + (lane >> 4);
    xchunk[i] = ((lane & 15) ^ (tok & 15)) * 16;
    xrow[i] = xq + min<int64_t>(t0 + tok, T - 1) * ld_q;
  }
  typedef uint32_t Bricks[kRF][6];  // per row fragment: mask words 0-1, code words 2-5
  auto load_bricks = [&](int64_t q, Bricks& bk) {
#pragma unroll
    for (int rf = 0; rf < kRF; ++rf) {
      const int64_t off = q << 6;  // slots advance by 64 per K step
      bk[rf][0] = bk[rf][1] = 0;
      if (has_mask) {
        const uint2 m = *reinterpret_cast<const uint2*>(mrow[rf] + off * 8);
        bk[rf][0] = m.x;
        bk[rf][1] = m.y;
      }
      bk[rf][2] = bk[rf][3] = bk[rf][4] = bk[rf][5] = 0;
      const uint8_t* c = crow[rf] + off * cbb;
      if constexpr (POS) {
        const uint4 v = *reinterpret_cast<const uint4*>(c);
        bk[rf][2] = v.x; bk[rf][3] = v.y; bk[rf][4] = v.z; bk[rf][5] = v.w;
      } else {
        for (int i = 0; i < cbb; ++i) bk[rf][2 + (i >> 2)] |= (uint32_t)c[i] << (8 * (i & 3));
      }
    }
  };
  auto load_x = [&](int64_t q) {  // step q's activation tile -> ring slot q % kXBufs
    int8_t* dst = xs0 + (int)(q % kXBufs) * kTileBytes;
    const int kq = (int)q * kQuadK;
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
      int8_t* d = dst + (wave * kXLoads + i) * 1024;
      if constexpr (XVEC) {
        // chunks past K read in-row data (K >= 16 here); the weights at those positions are 0
        const int k = min(kq + xchunk[i], K - 16);
        __builtin_amdgcn_global_load_lds((const void*)(xrow[i] + k), (lds_ptr)d, 16, 0, 0);
      } else {
        *reinterpret_cast<v4i*>(d + lane * 16) = load_x16<false>(xrow[i], kq + xchunk[i], K);
      }
    }
  };
  auto decode_slice = [&](const Bricks& bk, int rf, int j, uint32_t* out) {
    if constexpr (POS) {
      exp_word_to_i8(bk[rf][2 + j], out);
    } else {
      const uint32_t m[2] = {bk[rf][0], bk[rf][1]};
      const uint32_t c[4] = {bk[rf][2], bk[rf][3], bk[rf][4], bk[rf][5]};
      uint32_t tmp[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) tmp[i] = 0;
      decode_kept_brick(m, c, L.n, L.m, L.has_mask, tmp);
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = tmp[4 * j + i];
    }
  };

  v4i acc[kRF][CF];
#pragma unroll
  for (int rf = 0; rf < kRF; ++rf)
#pragma unroll
    for (int cf = 0; cf < CF; ++cf) acc[rf][cf] = v4i{0, 0, 0, 0};
  // Fragment read offsets: token cf*16 + t (t = lane % 16), global chunk 4*(lane/16) + j.
  const int t_l = lane & 15, g_l = lane >> 4;
  int boff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) boff[j] = t_l * kQuadK + (((4 * g_l + j) ^ t_l) * 16);
  // Vector-memory operations issued per step (activation pieces + brick loads).
  constexpr int kStepLoads = kXLoads + kRF;

  uint32_t a[kRF][16];
  Bricks b0, b1;
  load_bricks(0, b0);
  load_x(0);
  load_bricks(min<int64_t>(1, nq - 1), b1);
  load_x(min<int64_t>(1, nq - 1));
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // ring slots of steps 0 and 1 written
  __syncthreads();
#pragma unroll
  for (int rf = 0; rf < kRF; ++rf)
#pragma unroll
    for (int j = 0; j < 3; ++j) decode_slice(b0, rf, j, a[rf] + 4 * j);

  // Step q (its A slices 0-2 already decoded, its bricks in `bcur`):
  //   MFMA group 0 while decoding slice 3 of step q (bcur); then the loads of step q+2 go out
  //   (bricks into bcur, now free; activations into ring slot (q+2) % 3);
  //   MFMA group j (j = 1..3) while decoding slice j-1 of step q+1 (bnext) into the registers
  //   that group j-1 has finished with.
  // Activation fragments are read one MFMA batch ahead. Before the closing barrier each wave
  // waits for its own step-(q+1) activation pieces (issued during step q-1): only the kStepLoads
  // operations issued in this step may still be in flight.
  auto step = [&](int64_t q, Bricks& bcur, const Bricks& bnext, bool has_next) {
    const int8_t* xt = xs0 + (int)(q % kXBufs) * kTileBytes;
    const bool prefetch = q + 2 < nq;
    v4i bv = *reinterpret_cast<const v4i*>(xt + boff[0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int cf = 0; cf < CF; ++cf) {
        const int nj = cf + 1 < CF ? j : j + 1, ncf = cf + 1 < CF ? cf + 1 : 0;
        v4i bn = bv;
        if (nj < 4) bn = *reinterpret_cast<const v4i*>(xt + ncf * 16 * kQuadK + boff[nj]);
#pragma unroll
        for (int rf = 0; rf < kRF; ++rf) acc[rf][cf] = mfma16(a[rf] + 4 * j, bv, acc[rf][cf]);
        bv = bn;
      }
      if (j == 0) {
#pragma unroll
        for (int rf = 0; rf < kRF; ++rf) decode_slice(bcur, rf, 3, a[rf] + 12);
      } else if (has_next) {
#pragma unroll
        for (int rf = 0; rf < kRF; ++rf) decode_slice(bnext, rf, j - 1, a[rf] + 4 * (j - 1));
      }
#pragma unroll
      for (int cf = 0; cf < CF; ++cf) {
        __builtin_amdgcn_sched_group_barrier(0x008, kRF, 0);        // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 2 + 2 * kRF, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);          // LDS read
      }
      if (j == 0 && prefetch) {
        load_bricks(q + 2, bcur);
        load_x(q + 2);
      }
    }
    if (prefetch && POS && XVEC) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kStepLoads));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    __syncthreads();
  };
  int64_t q = 0;
  for (; q + 2 < nq; q += 2) {
    step(q, b0, b1, true);
    step(q + 1, b1, b0, true);
  }
  if (q + 1 < nq) {
    step(q, b0, b1, true);
    step(q + 1, b1, b0, false);
  } else {
    step(q, b0, b1, false);
  }

  const float gamma = gamma_p[0];
  // Each lane holds 4 consecutive rows of one token per (rf, cf): one 16-byte store when the
  // output rows are 16-byte aligned and all 4 rows exist.
  const bool vec_out = (((uintptr_t)y | (uintptr_t)(ld_y * 4)) & 15) == 0;
#pragma unroll
  for (int cf = 0; cf < CF; ++cf) {
    const int64_t t = t0 + cf * 16 + t_l;
    if (t >= T) continue;
    const float step_t = out_kind == SBN_OUT_F32 ? absmax[t] / 127.0f : 0.0f;
#pragma unroll
    for (int rf = 0; rf < kRF; ++rf) {
      const int64_t r0 = (rb0 + rf) * 16 + 4 * g_l;
      const v4i v = acc[rf][cf];
      if (vec_out && r0 + 4 <= L.n_out) {
        if (out_kind == SBN_OUT_I32_ACC) {
          *reinterpret_cast<v4i*>(reinterpret_cast<int32_t*>(y) + t * ld_y + r0) = v;
        } else {
          float4 f;
          f.x = __fmul_rn(__fmul_rn((float)v[0], gamma), step_t);
          f.y = __fmul_rn(__fmul_rn((float)v[1], gamma), step_t);
          f.z = __fmul_rn(__fmul_rn((float)v[2], gamma), step_t);
          f.w = __fmul_rn(__fmul_rn((float)v[3], gamma), step_t);
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + t * ld_y + r0) = f;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (r0 + i < L.n_out) store_out(y, ld_y, out_kind, t, r0 + i, v[i], gamma, step_t);
      }
    }
  }
}

template <int CF>
constexpr size_t gemm_smem_bytes() {
  return (size_t)kXBufs * CF * 16 * kQuadK;
}

// Raises a kernel's dynamic-LDS limit once per process (gfx950 has 160 KB of LDS per CU).
template <typename K>
hipError_t allow_smem(K kernel, size_t bytes) {
  static size_t done = 0;
  if (bytes <= done) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done = bytes;
  return e;
}

template <bool POS, bool XVEC>
hipError_t launch_pattern(const sbn_packed* h, const int8_t* xq, int64_t ld_q,
                          const float* absmax, int64_t T, void* y, int64_t ld_y, int out_kind,
                          hipStream_t s) {
  const Layout& L = h->L;
  if (T <= 16) {
    const size_t xs_bytes = (size_t)T * kGemvXStride;
    if (T <= 4) {
      hipError_t e = allow_smem(bitlinear_gemv<POS, XVEC, 1>, xs_bytes);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((bitlinear_gemv<POS, XVEC, 1>), dim3((unsigned)L.row_blocks),
                         dim3(256), xs_bytes, s, h->mask, h->codes, L, h->gamma, xq, ld_q, absmax,
                         T, y, ld_y, out_kind);
    } else {
      hipError_t e = allow_smem(bitlinear_gemv<POS, XVEC, 2>, xs_bytes);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((bitlinear_gemv<POS, XVEC, 2>),
                         dim3((unsigned)((L.row_blocks + 1) / 2)), dim3(256), xs_bytes, s, h->mask,
                         h->codes, L, h->gamma, xq, ld_q, absmax, T, y, ld_y, out_kind);
    }
    return hipGetLastError();
  }
  constexpr int CF = kGemmCF;
  constexpr size_t smem = gemm_smem_bytes<CF>();
  hipError_t e = allow_smem(bitlinear_gemm<POS, CF, XVEC>, smem);
  if (e != hipSuccess) return e;
  const int64_t gx = (L.row_blocks + kGemmWaves * kRF - 1) / (kGemmWaves * kRF);
  const int64_t gy = (T + CF * 16 - 1) / (CF * 16);
  hipLaunchKernelGGL((bitlinear_gemm<POS, CF, XVEC>), dim3((unsigned)(gx * gy)),
                     dim3(kGemmThreads),
                     smem, s, h->mask, h->codes, L, h->gamma, xq, ld_q, absmax, T, y, ld_y,
                     out_kind, (int)gx, (int)gy);
  return hipGetLastError();
}

template <bool POS>
hipError_t launch_pattern_x(const sbn_packed* h, const int8_t* xq, int64_t ld_q,
                            const float* absmax, int64_t T, void* y, int64_t ld_y, int out_kind,
                            hipStream_t s) {
  const bool xvec = ((uintptr_t)xq % 16 == 0) && (ld_q % 16 == 0) && (h->L.K % 16 == 0);
  if (xvec) return launch_pattern<POS, true>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
  return launch_pattern<POS, false>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
}

}  // namespace

hipError_t launch_bitlinear(const sbn_packed* h, const int8_t* xq, int64_t ld_q,
                            const float* absmax, int64_t T, void* y, int64_t ld_y, int out_kind,
                            hipStream_t s) {
  const Layout& L = h->L;
  if (L.n_out == 0 || T == 0) return hipSuccess;
  if (L.positional) return launch_pattern_x<true>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
  return launch_pattern_x<false>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
}

}  // namespace sbn
