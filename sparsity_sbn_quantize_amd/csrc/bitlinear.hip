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
//   GEMV (T <= 16): one workgroup per 16-row fragment row, its waves split K (one to three
//   256-K quads each, in batches past 48 quads with int8 input); operands go straight from memory
//   into MFMA registers and the waves' sums meet once in LDS. With bf16 input (T <= 4, K <= 12288)
//   every workgroup also quantizes (optionally after a parameter-free LayerNorm) the activations
//   it needs; for one token it can also add the k:256 outlier term.
//   GEMM (T > 16): a workgroup computes 256 rows x 128 (or 64) tokens; the activation tile of each
//   K step is staged in LDS and shared by the waves; 2:4 runs on the structured-sparse MFMA.
#include <algorithm>

#include "gemv.hpp"

namespace sbn {
namespace {

// GEMM (T > 16): a workgroup of W = 4 waves computes 256 rows x 16 CF tokens (CF = 8: 128 tokens;
// CF = 4: 64); wave w owns 4 row fragments (64 rows) and all the tile's tokens. Two workgroups
// share a CU (two waves per SIMD), so one wave's decode and LDS traffic overlap the other's MFMAs.
// Launches with many 128-token tiles take W = 8 waves on 512 rows instead (one workgroup per
// CU, still two waves per SIMD): each step's activation tile then goes to LDS once for 512 rows
// instead of once per 256, and the global -> LDS transfers of the activation tiles were what
// bounded the K loop (timing copies with half of those transfers left out ran 9-18% faster).
// K advances 256 per step. Each step's activation tile goes global -> LDS directly
// (global_load_lds, no registers) into a 2-slot ring, one step ahead, laid out so that every
// fragment read is free of bank conflicts. K slice j+1 of the wave's row fragments is decoded while
// the MFMAs of slice j run (two A register sets); bricks are loaded one step ahead. One barrier per
// step. CF = 8 reuses each decoded slice for twice as many MFMAs; CF = 4 doubles the tile count of
// launches that would otherwise leave CUs idle (see the launcher).
constexpr int kGemmWaves = 4;
constexpr int kRF = 4;                                  // 16-row fragments per wave
constexpr int kGemmRowBlocks = kGemmWaves * kRF;        // 16 row fragments (256 rows) per tile
constexpr int kXBufs = 2;                               // activation ring depth

// LDS of a CF tile: the activation ring, then the tile's a'_t (one float per token).
constexpr size_t gemm_smem(int cf) { return (size_t)kXBufs * cf * 16 * kQuadK + cf * 16 * 4; }

// Split-K (two workgroups per tile, each half of K) for launches that have few tiles even at CF = 4. The halves of a
// tile are adjacent in the XCD order (same L2). Per tile and wave, the first half to finish
// stores its int32 partial sums in the tile's region of y and publishes them; the second waits
// (a bounded spin: the first is already past its main loop, so it is running), adds the partial
// and writes the result. Integer sums make the result independent of the order. Each (tile, wave)
// slot has two words in the weight handle, never reset: an arrival counter (each launch adds 2,
// so the old value's parity says which half came first and its half is the slot's launch count)
// and the launch count the partial sums were last published for; the second half waits for its
// own launch's count, so a value left by an earlier launch (or by a half that gave up waiting)
// never matches, and graph replays need no host-side state. A half that gives up adds 1 to the
// handle's give-up counter (sbn_packed_query) and stores a wrong tile. Arrivals of two launches
// that share a handle must not interleave, so such calls must be ordered (one stream, or
// synchronized). Sharing tiles more
// widely (a contiguous share of all tiles' K steps for every resident workgroup, or three
// workgroups per tile) was measured slower on the 2048- and 8192-token shapes: the partial sums
// then move about as many bytes as the fp32 output, all at the same moment.
constexpr int kOutPolicy = 1 | 2 | 16;  // buffer cache-policy bits sc0 | nt | sc1: output stores
constexpr int kSplitMaxTiles = 256;    // split when a launch has at most this many tiles
constexpr int kWideMinTiles = 200;     // 512-row tiles when a launch has at least this many
constexpr int kOneRoundTiles = 256;    // 8-wave workgroups that run at once (one per CU)
static_assert(kGemmSyncInts >= kSplitMaxTiles * 4 * 2, "split-K words of the handle");

template <int FORM, bool XVEC, int CF, int W>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bitlinear_gemm(const uint8_t* __restrict__ mask_plane, const uint8_t* __restrict__ code_plane,
                    Layout L, const float* __restrict__ gamma_p, const int8_t* __restrict__ xq,
                    int64_t ld_q, const float* __restrict__ absmax, int64_t T,
                    void* __restrict__ y, int64_t ld_y, int out_kind, int tiles_n, int tiles_t,
                    int ksplit, uint32_t* __restrict__ sync, int spin_limit, int publish) {
  constexpr int kGemmCF = CF;                             // 16-token fragments per tile
  constexpr int kGemmTok = CF * 16;                       // tokens per tile
  constexpr int kTileBytes = kGemmTok * kQuadK;           // one step's activation tile
  constexpr int kXLoads = kGemmTok * 16 / (W * 64);       // 16-byte pieces per thread per step
  static_assert(kXLoads * W * 64 == kGemmTok * 16, "the waves share a step's loads evenly");
  constexpr size_t kRing = (size_t)kXBufs * kTileBytes;
  constexpr bool POS = FORM != kFormKept;  // 16 code bytes per lane and quad
  constexpr bool SP = FORM == kFormSparse24;
  constexpr int kBW = POS ? 4 : 6;  // brick words in registers: codes, or mask (2) + codes (4)
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int8_t* const xs0 = reinterpret_cast<int8_t*>(smem);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // wave-uniform
  const int lane = threadIdx.x & 63;
  const int lin = xcd_order((int)gridDim.x, (int)blockIdx.x);
  const int tile_lin = lin / ksplit, half = lin % ksplit;
  int tile_n, tile_t;
  grouped_tile(tile_lin, tiles_n, tiles_t, tile_n, tile_t);
  const int64_t rb0 = ((int64_t)tile_n * W + wave) * kRF;
  const int64_t t0 = (int64_t)tile_t * kGemmTok;
  const int nq = (int)L.quads;
  const int qb = nq * half / ksplit, qe = nq * (half + 1) / ksplit;  // this workgroup's K steps
  const int K = (int)L.K;
  const int cbb = POS ? 16 : L.code_brick_bytes;

  // Brick addresses: a wave-uniform base plus lane * (brick bytes); row fragment rf and step q are
  // uniform offsets. Stored row fragments are padded to a multiple of 16, so every tile's rows
  // exist (the padding is zero and its results are never stored).
  const int64_t frag0 = rb0 * nq;
  const uint8_t* const cbase = code_plane + (frag0 << 6) * cbb;
  const uint8_t* const mbase = POS ? nullptr : mask_plane + (frag0 << 6) * 8;
  const int64_t rf_stride = (int64_t)nq << 6;  // slots per row fragment
  // Positional bricks go through a buffer resource (base in scalar registers, one 32-bit lane
  // offset): every offset a tile uses is below kRF * nq * 1024 bytes <= 2 MB. The stored plane
  // ends at a multiple of 256 rows; with 512-row tiles the waves of a last tile's second half lie
  // wholly past it, and their resource is empty (every brick reads zero).
  const __amdgpu_buffer_rsrc_t crsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)cbase, (short)0, rb0 < L.row_blocks_pad ? 0x7FFFFFFF : 0, kBufDword3);
  const int lane_c = lane * cbb;
  // Activation pieces are read relative to the tile's first token row. The aligned path reads
  // through buffer resources whose range ends with the last activation row: pieces of tokens past
  // T, or of the last row past K, read as zero (elsewhere a piece past K reads in-row data,
  // harmless because the weights there are zero). Tokens past T are never stored.
  const int8_t* const xt0 = xq + t0 * ld_q;
  const int64_t x_extent = (T - 1 - t0) * ld_q + K;  // bytes from xt0 to the end of row T-1
  // Activation tile layout in LDS: [16-token group cf][K chunk c (16 bytes)][token t], i.e. the
  // 16-byte piece of token cf*16 + t at K chunk c sits at cf*4096 + c*256 + t*16. The fragment
  // read of (slice j, group cf) then has the 16 lanes of each lane group g read 256 contiguous
  // bytes (chunk 4g + j of tokens 0..15), which gfx950's LDS serves without bank conflicts. Wave
  // instruction ii loads group ii / 4, chunks 4 (ii % 4) .. +3: lane l takes token l % 16, chunk
  // 4 (ii % 4) + l / 16, i.e. 64 contiguous bytes of each of 16 token rows, and lands at
  // 1 KB-block ii + 16 l as the layout requires. The per-instruction part of the address is
  // uniform (folded into the instruction's buffer resource); the lane part is one offset.
  const int xlane = (lane & 15) * (int)ld_q + (lane >> 4) * 16;
  // fragment read offset: chunk 4g (+ j) of token t for the dense MFMA; chunk g (+ 4, + 8 ...)
  // for the sparse MFMA (g = lane / 16, t = lane % 16)
  const int rlane = (lane >> 4) * (SP ? 256 : 1024) + (lane & 15) * 16;
  auto load_x = [&](int q, int slot) {  // step q's activation tile -> ring slot
    int8_t* dst = xs0 + slot * kTileBytes + wave * (kXLoads * 1024);
    const int kq = q * kQuadK;
    if constexpr (XVEC) {
      // One buffer resource per step, based at the step's K offset of the tile's first token row,
      // whose range ends with row T-1: pieces of tokens past T, or of the last row past K, read as
      // zero (elsewhere a piece past K reads in-row data, harmless because the weights there are
      // zero). Tokens past T are never stored. The piece's place in the tile is a lane offset
      // (below 128 ld_q + 256 < 2^31: the launcher takes this path for ld_q < 2^24). Same-box
      // A/B against one resource per load (8 per wave and step, 16 scalar instructions each):
      // 6912 -> 2560 at T = 2048 46.1 -> 43.7 us, the other shapes unchanged.
      const int64_t left = x_extent - kq;
      const int nrec = left <= 0 ? 0 : (left > 0x7FFFFFFF ? 0x7FFFFFFF : (int)left);
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc((void*)(xt0 + kq), (short)0, nrec, kBufDword3);
      const int ldq = (int)ld_q;
#pragma unroll
      for (int i = 0; i < kXLoads; ++i) {
        const int ii = wave * kXLoads + i, cf = ii >> 2, c0 = (ii & 3) * 4;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)(dst + i * 1024), 16,
                                                 xlane + cf * 16 * ldq + c0 * 16, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kXLoads; ++i) {
        const int ii = wave * kXLoads + i, cf = ii >> 2, c0 = (ii & 3) * 4;
        const int tok = cf * 16 + (lane & 15), c = c0 + (lane >> 4);
        const int8_t* row = xq + min<int64_t>(t0 + tok, T - 1) * ld_q;
        *reinterpret_cast<v4i*>(dst + i * 1024 + lane * 16) = load_x16<false>(row, kq + c * 16, K);
      }
    }
  };
  typedef uint32_t Bricks[kRF][kBW];
  auto load_bricks = [&](int q, Bricks& bk) {
#pragma unroll
    for (int rf = 0; rf < kRF; ++rf) {
      const int64_t slot0 = rf * rf_stride + ((int64_t)q << 6);  // uniform
      if constexpr (POS) {
        const v4i v = __builtin_amdgcn_raw_buffer_load_b128(crsrc, lane_c, (int)(slot0 * 16), 0);
        bk[rf][0] = (uint32_t)v[0]; bk[rf][1] = (uint32_t)v[1];
        bk[rf][2] = (uint32_t)v[2]; bk[rf][3] = (uint32_t)v[3];
      } else {
        bk[rf][0] = bk[rf][1] = 0;
        if (L.has_mask) {
          const uint2 m = *reinterpret_cast<const uint2*>(mbase + (slot0 + lane) * 8);
          bk[rf][0] = m.x;
          bk[rf][1] = m.y;
        }
        bk[rf][2] = bk[rf][3] = bk[rf][4] = bk[rf][5] = 0;
        const uint8_t* c = cbase + slot0 * cbb + lane_c;
        for (int i = 0; i < cbb; ++i) bk[rf][2 + (i >> 2)] |= (uint32_t)c[i] << (8 * (i & 3));
      }
    }
  };
  typedef uint32_t ASlice[kRF][4];
  // A operand of MFMA slice j (dense forms) or of 128-K block j (sparse form: the block's kept
  // weights; its index word stays in the brick registers).
  auto decode_slice = [&](const Bricks& bk, int j, ASlice& out) {
#pragma unroll
    for (int rf = 0; rf < kRF; ++rf) {
      if constexpr (SP) {
        exp_word_to_i8(bk[rf][2 * j], out[rf]);
      } else if constexpr (POS) {
        exp_word_to_i8(bk[rf][j], out[rf]);
      } else {
        const uint32_t m[2] = {bk[rf][0], bk[rf][1]};
        const uint32_t c[4] = {bk[rf][2], bk[rf][3], bk[rf][4], bk[rf][5]};
        uint32_t tmp[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) tmp[i] = 0;
        decode_kept_brick(m, c, L.n, L.m, L.has_mask, tmp);
#pragma unroll
        for (int i = 0; i < 4; ++i) out[rf][i] = tmp[4 * j + i];
      }
    }
  };

  v4i acc[kRF][kGemmCF];
#pragma unroll
  for (int rf = 0; rf < kRF; ++rf)
#pragma unroll
    for (int cf = 0; cf < kGemmCF; ++cf) acc[rf][cf] = v4i{0, 0, 0, 0};
  const int t_l = lane & 15, g_l = lane >> 4;

  // The tile's activation scales go to LDS with the first operands. The epilogue reads them from
  // there: a load from memory at that point would wait (vmcnt) for the stores already issued,
  // which made each 16-token group's stores wait for the previous group's.
  float* const am_s = reinterpret_cast<float*>(smem + kRing);
  float am_v = 0.0f;
  if (out_kind == SBN_OUT_F32 && (int)threadIdx.x < kGemmTok)
    am_v = absmax[min<int64_t>(t0 + threadIdx.x, T - 1)];
  Bricks b0, b1;
  ASlice a0, a1;
  load_bricks(qb, b0);
  load_x(qb, 0);
  load_bricks(min(qb + 1, nq - 1), b1);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // ring slot of step 0 written
  if ((int)threadIdx.x < kGemmTok) am_s[threadIdx.x] = am_v;
  __syncthreads();
  decode_slice(b0, 0, a0);

  // Step q (slice 0 of its A already decoded into a0, its bricks in bcur, step q+1's in bnext):
  // the activation tile of step q+1 goes out first; MFMA group j (slice j, 4 row fragments x 8
  // token fragments) runs while slice j+1 is decoded into the other A set (slice 0 of step q+1
  // during group 3); after group 3 the bricks of step q+2 are loaded into bcur. Before the
  // closing barrier each wave waits for its step-(q+1) activation pieces: only the brick loads
  // issued after them may still be in flight.
  // Schedule of a dense step: per token fragment, its 4 MFMAs, 24 / CF VALU instructions of the
  // next slice's decode, one LDS read. Same-process A/B of the VALU count per group (CF = 8):
  // 3 against 5 took 6912 -> 2560 at T = 2048 from 50.5 to 49.0 us and the 7B down projection at
  // T = 8192 from 275 to 273 us; 4, 6 and 8 were no better; the other shapes did not change.
  auto step = [&](int q, int slot, Bricks& bcur, const Bricks& bnext) {
    // Unconditional, so that the step is straight-line code and the compiler's counter waits for
    // the brick registers stay exact: past the last step the tile's range is empty (reads are
    // zero) and the slot it fills is never read.
    load_x(q + 1, slot ^ 1);
    __builtin_amdgcn_sched_barrier(0);  // the tile loads go out before this step's MFMAs
    const int8_t* xt = xs0 + slot * kTileBytes + rlane;
    v4i bv = *reinterpret_cast<const v4i*>(xt);
    if constexpr (POS) {
      // Fenced groups: group (j, cf) issues the LDS read of the next group's B first, then its 4
      // MFMAs, then its share of the next slice's decode (2 kRF half-words over CF groups), and
      // nothing crosses the fence after it, so every B read is one group ahead of its MFMAs.
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ASlice& cur = (j & 1) ? a1 : a0;
        ASlice& nxt = (j & 1) ? a0 : a1;
        const Bricks& src = j < 3 ? bcur : bnext;
        const int sj = j < 3 ? j + 1 : 0;
#pragma unroll
        for (int cf = 0; cf < kGemmCF; ++cf) {
          const int nj = cf + 1 < kGemmCF ? j : j + 1, ncf = cf + 1 < kGemmCF ? cf + 1 : 0;
          v4i bn = bv;
          if (nj < 4) bn = *reinterpret_cast<const v4i*>(xt + ncf * 4096 + nj * 256);
#pragma unroll
          for (int rf = 0; rf < kRF; ++rf) acc[rf][cf] = mfma16(cur[rf], bv, acc[rf][cf]);
#pragma unroll
          for (int p = cf * 2 * kRF / kGemmCF; p < (cf + 1) * 2 * kRF / kGemmCF; ++p)
            exp_word_half_to_i8(src[p >> 1][sj], p & 1, nxt[p >> 1][2 * (p & 1)],
                                nxt[p >> 1][2 * (p & 1) + 1]);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // LDS read
          __builtin_amdgcn_sched_group_barrier(0x008, kRF, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);   // VALU
          __builtin_amdgcn_sched_barrier(0);
          bv = bn;
        }
      }
    } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ASlice& cur = (j & 1) ? a1 : a0;
      ASlice& nxt = (j & 1) ? a0 : a1;
#pragma unroll
      for (int cf = 0; cf < kGemmCF; ++cf) {
        const int nj = cf + 1 < kGemmCF ? j : j + 1, ncf = cf + 1 < kGemmCF ? cf + 1 : 0;
        v4i bn = bv;
        if (nj < 4) bn = *reinterpret_cast<const v4i*>(xt + ncf * 4096 + nj * 256);
#pragma unroll
        for (int rf = 0; rf < kRF; ++rf) acc[rf][cf] = mfma16(cur[rf], bv, acc[rf][cf]);
        bv = bn;
      }
      if (j < 3) {
        decode_slice(bcur, j + 1, nxt);
      } else {
        decode_slice(bnext, 0, nxt);
      }
#pragma unroll
      for (int cf = 0; cf < kGemmCF; ++cf) {
        __builtin_amdgcn_sched_group_barrier(0x008, kRF, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 24 / CF, 0);  // VALU (A/B: 3 per group)
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // LDS read
      }
    }
    }
    load_bricks(min(q + 2, nq - 1), bcur);
    if (POS && XVEC) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kRF));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    __syncthreads();
  };
  // Sparse 2:4 step: two 128-K blocks; block 0's 32 structured-sparse MFMAs run while block 1's
  // kept weights are decoded, block 1's while the next step's block 0 is decoded. Each B operand
  // is two 16-byte reads (chunks g and g + 4 of the block).
  auto step_sp = [&](int q, int slot, Bricks& bcur, const Bricks& bnext) {
    load_x(q + 1, slot ^ 1);
    __builtin_amdgcn_sched_barrier(0);  // the tile loads go out before this step's MFMAs
    const int8_t* xt = xs0 + slot * kTileBytes + rlane;
    v4i blo = *reinterpret_cast<const v4i*>(xt);
    v4i bhi = *reinterpret_cast<const v4i*>(xt + 1024);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      ASlice& cur = blk ? a1 : a0;
      ASlice& nxt = blk ? a0 : a1;
      const Bricks& src = blk == 0 ? bcur : bnext;
      const int sj = blk == 0 ? 1 : 0;
#pragma unroll
      for (int cf = 0; cf < kGemmCF; ++cf) {
        const int nb = cf + 1 < kGemmCF ? blk : blk + 1, ncf = cf + 1 < kGemmCF ? cf + 1 : 0;
        v4i nlo = blo, nhi = bhi;
        if (nb < 2) {
          nlo = *reinterpret_cast<const v4i*>(xt + ncf * 4096 + nb * 2048);
          nhi = *reinterpret_cast<const v4i*>(xt + ncf * 4096 + nb * 2048 + 1024);
        }
#pragma unroll
        for (int rf = 0; rf < kRF; ++rf)
          acc[rf][cf] = smfmac16(cur[rf], blo, bhi, bcur[rf][2 * blk + 1], acc[rf][cf]);
        // fenced as the dense step: next group's B reads first, then the MFMAs, then this group's
        // share of the next block's decode
#pragma unroll
        for (int p = cf * 2 * kRF / kGemmCF; p < (cf + 1) * 2 * kRF / kGemmCF; ++p)
          exp_word_half_to_i8(src[p >> 1][2 * sj], p & 1, nxt[p >> 1][2 * (p & 1)],
                              nxt[p >> 1][2 * (p & 1) + 1]);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);    // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, kRF, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);   // VALU
        __builtin_amdgcn_sched_barrier(0);
        blo = nlo;
        bhi = nhi;
      }
    }
    load_bricks(min(q + 2, nq - 1), bcur);
    if (XVEC) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kRF));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    __syncthreads();
  };
  int q = qb;
  if constexpr (SP) {
    for (; q + 1 < qe; q += 2) {
      step_sp(q, 0, b0, b1);
      step_sp(q + 1, 1, b1, b0);
    }
    if (q < qe) step_sp(q, 0, b0, b1);
  } else {
    for (; q + 1 < qe; q += 2) {
      step(q, 0, b0, b1);
      step(q + 1, 1, b1, b0);
    }
    if (q < qe) step(q, 0, b0, b1);
  }

  // Each lane holds 4 consecutive rows of one token per (rf, cf): one 16-byte access when the
  // output rows are 16-byte aligned and all 4 rows exist.
  const bool vec_out = (((uintptr_t)y | (uintptr_t)(ld_y * 4)) & 15) == 0;
  if (ksplit > 1) {
    // Every access of the handshake is coherent across the XCDs' L2 caches on its own (sc1:
    // relaxed agent-scope atomics for the flags, sc1 buffer accesses for the partial sums);
    // acquire/release fences would instead write back or invalidate whole L2s. Order: the
    // partial sums are stored, the wave waits until its stores have completed, then publishes
    // its launch count; the other half reads the partial sums only after it has seen that count.
    constexpr int kSc1 = 1 << 4;  // buffer cache-policy bit: sc1
    uint32_t* const arrive = sync + 2 * ((int64_t)tile_lin * W + wave);
    uint32_t* const ready = arrive + 1;
    const __amdgpu_buffer_rsrc_t yr =
        __builtin_amdgcn_make_buffer_rsrc(y, (short)0, 0x7FFFFFFF, kBufDword3);
    uint32_t old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = (uint32_t)__builtin_amdgcn_readfirstlane((int)old);
    // this launch's count on the slot (>= 1); the first arrival found an even count of arrivals
    const uint32_t gen = (old >> 1) + 1u;
    if ((old & 1u) == 0) {
#pragma unroll
      for (int cf = 0; cf < kGemmCF; ++cf) {
        const int64_t t = t0 + cf * 16 + t_l;
        if (t >= T) continue;
#pragma unroll
        for (int rf = 0; rf < kRF; ++rf) {
          const int64_t r0 = (rb0 + rf) * 16 + 4 * g_l;
          const int off = (int)((t * ld_y + r0) * 4);
          if (vec_out && r0 + 4 <= L.n_out) {
            __builtin_amdgcn_raw_buffer_store_b128(acc[rf][cf], yr, off, 0, kSc1);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (r0 + i < L.n_out)
                __builtin_amdgcn_raw_buffer_store_b32(acc[rf][cf][i], yr, off + 4 * i, 0, kSc1);
          }
        }
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);  // the partial sums have been written
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (lane == 0 && publish)
        __hip_atomic_store(ready, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    if (lane == 0) {
      int it = 0;
      for (; it < spin_limit; ++it) {
        if (__hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen) break;
        __builtin_amdgcn_s_sleep(2);
      }
      if (it == spin_limit)
        __hip_atomic_fetch_add(sync + kGemmSyncInts, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
    for (int cf = 0; cf < kGemmCF; ++cf) {
      const int64_t t = t0 + cf * 16 + t_l;
      if (t >= T) continue;
#pragma unroll
      for (int rf = 0; rf < kRF; ++rf) {
        const int64_t r0 = (rb0 + rf) * 16 + 4 * g_l;
        const int off = (int)((t * ld_y + r0) * 4);
        if (vec_out && r0 + 4 <= L.n_out) {
          acc[rf][cf] += __builtin_amdgcn_raw_buffer_load_b128(yr, off, 0, kSc1);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (r0 + i < L.n_out)
              acc[rf][cf][i] += __builtin_amdgcn_raw_buffer_load_b32(yr, off + 4 * i, 0, kSc1);
        }
      }
    }
  }

  const float gamma = gamma_p[0];
  // Vector stores go through a buffer resource based at the tile's first token row (offsets below
  // kGemmTok * ld_y * 4 < 2^31 whenever ld_y < 2^22; otherwise plain global stores), written
  // through with the system-scope non-temporal policy. Same-process A/B against plain global
  // stores: 2560 -> 6912 at T = 2048 42.1 -> 39.6 us (2:4: 35.5 -> 32.6), 6912 -> 2560 52.0 ->
  // 50.6, the 7B FFN shapes at T = 8192 unchanged; without sc1 (sc0 nt) it was slower than plain.
  const bool ybuf = ld_y < (int64_t{1} << 22);
  const __amdgpu_buffer_rsrc_t yo = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<int32_t*>(y) + t0 * ld_y, (short)0, 0x7FFFFFFF, kBufDword3);
#pragma unroll
  for (int cf = 0; cf < kGemmCF; ++cf) {
    const int64_t t = t0 + cf * 16 + t_l;
    if (t >= T) continue;
    const float step_t = am_s[cf * 16 + t_l] / 127.0f;
#pragma unroll
    for (int rf = 0; rf < kRF; ++rf) {
      const int64_t r0 = (rb0 + rf) * 16 + 4 * g_l;
      const v4i v = acc[rf][cf];
      if (vec_out && r0 + 4 <= L.n_out) {
        v4i o = v;
        if (out_kind != SBN_OUT_I32_ACC) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            o[i] = (int)__float_as_uint(__fmul_rn(__fmul_rn((float)v[i], gamma), step_t));
        }
        if (ybuf) {
          __builtin_amdgcn_raw_buffer_store_b128(o, yo, (int)(((t - t0) * ld_y + r0) * 4), 0,
                                                 kOutPolicy);
        } else {
          *reinterpret_cast<v4i*>(reinterpret_cast<int32_t*>(y) + t * ld_y + r0) = o;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (r0 + i < L.n_out) store_out(y, ld_y, out_kind, t, r0 + i, v[i], gamma, step_t);
      }
    }
  }
}

// Launches the bf16-input GEMV (the int8-input GEMV is launched from gemv_i8.hip) with
// W = ceil(quads / 3) waves and Q = ceil(quads / W) quads per wave, so that its workgroup barriers
// wait for fewer waves (same-process A/B on the 2560 -> 6912 shape, one-kernel step at T = 1: 4.45 us at three
// quads per wave, 4.72 at one, 4.60 at two, 4.65 at four, 4.93 at five; with the LayerNorm 6.46 vs
// 7.56). Rechecked with non-temporal brick loads: three quads per wave stays fastest on the
// decode shape (4.2 vs 4.4 at two, 4.6 at one) and on 6912 -> 2560; on 4096 -> 11008 at 2:4 (16
// quads) two per wave measured faster (5.48 vs 5.85 us), so no single count fits every shape. The
// int8 kernel, which has no barrier before its products, is fastest at one quad per wave (3.77 vs
// 3.85 us at two).
template <int FORM, bool FUSED, bool XVEC>
hipError_t launch_gemv(const sbn_packed* h, const void* x, int64_t ld_x, int8_t* xq_out,
                       int64_t ld_q, float* absmax, int64_t T, void* y, int64_t ld_y,
                       int out_kind, float ln_eps, hipStream_t s) {
  const Layout& L = h->L;
  const int W =
      (int)std::min<int64_t>(kGemvMaxWaves, FUSED ? (L.quads + kGemvMaxQ - 1) / kGemvMaxQ : L.quads);
  const int Q = (int)((L.quads + W - 1) / W);
#define SBN_GEMV(QQ, LNV, XB)                                                                 \
  hipLaunchKernelGGL((bitlinear_gemv<FORM, FUSED, XVEC, QQ, LNV, XB>),                           \
                     dim3((unsigned)L.row_blocks), dim3(64 * W), 0, s, h->mask,                  \
                     compact_form(FORM) ? h->cplane : h->codes, L,                                 \
                     h->gamma_out(), x, ld_x, xq_out, ld_q, absmax, T, y, ld_y, out_kind, ln_eps)
#define SBN_GEMV_Q(QQ)                                                                        \
  if constexpr (FUSED) {                                                                      \
    if (ln_eps > 0.0f) SBN_GEMV(QQ, FUSED, false);                                            \
    else if (XVEC && T == 1) SBN_GEMV(QQ, false, FUSED);                                      \
    else SBN_GEMV(QQ, false, false);                                                          \
  } else {                                                                                    \
    if (T <= kFusedMaxT) SBN_GEMV(QQ, false, !FUSED); else SBN_GEMV(QQ, false, false);        \
  }
  if (Q == 1) {
    SBN_GEMV_Q(1);
  } else if (Q == 2) {
    SBN_GEMV_Q(2);
  } else {
    SBN_GEMV_Q(3);
  }
#undef SBN_GEMV_Q
#undef SBN_GEMV
  return hipGetLastError();
}

// The grouped one-kernel step (members as in bitlinear_gemv_group), with the wave and quad counts
// of launch_gemv's one-kernel step.
template <int FORM, bool XVEC>
hipError_t launch_gemv_group_fused(const GemvGroup& G, int blocks, const Layout& L,
                                   const uint16_t* x, int64_t ld_x, int8_t* xq_out, int64_t ld_q,
                                   float* absmax, int64_t T, int out_kind, float ln_eps,
                                   hipStream_t s) {
  const int W = (int)std::min<int64_t>(kGemvMaxWaves, (L.quads + kGemvMaxQ - 1) / kGemvMaxQ);
  const int Q = (int)((L.quads + W - 1) / W);
#define SBN_GEMVG(QQ, LNV, XB)                                                                \
  hipLaunchKernelGGL((bitlinear_gemv_group<FORM, true, XVEC, QQ, LNV, XB>), dim3((unsigned)blocks), \
                     dim3(64 * W), 0, s, G, L, static_cast<const void*>(x), ld_x, xq_out, ld_q,  \
                     absmax, T, out_kind, ln_eps)
#define SBN_GEMVG_Q(QQ)                                                                       \
  do {                                                                                        \
    if (ln_eps > 0.0f) SBN_GEMVG(QQ, true, false);                                            \
    else if (XVEC && T == 1) SBN_GEMVG(QQ, false, true);                                      \
    else SBN_GEMVG(QQ, false, false);                                                         \
  } while (0)
  if (Q == 1) {
    SBN_GEMVG_Q(1);
  } else if (Q == 2) {
    SBN_GEMVG_Q(2);
  } else {
    SBN_GEMVG_Q(3);
  }
#undef SBN_GEMVG_Q
#undef SBN_GEMVG
  return hipGetLastError();
}

// The GEMV on the compact plane, by group size.
template <bool FUSED, bool XVEC>
hipError_t launch_gemv_compact(const sbn_packed* h, const void* x, int64_t ld_x, int8_t* xq_out,
                               int64_t ld_q, float* absmax, int64_t T, void* y, int64_t ld_y,
                               int out_kind, float ln_eps, hipStream_t s) {
  if (h->L.m == 4)
    return launch_gemv<kFormCompact4, FUSED, XVEC>(h, x, ld_x, xq_out, ld_q, absmax, T, y, ld_y,
                                                   out_kind, ln_eps, s);
  if (h->L.m == 8)
    return launch_gemv<kFormCompact8, FUSED, XVEC>(h, x, ld_x, xq_out, ld_q, absmax, T, y, ld_y,
                                                   out_kind, ln_eps, s);
  return launch_gemv<kFormCompact16, FUSED, XVEC>(h, x, ld_x, xq_out, ld_q, absmax, T, y, ld_y,
                                                  out_kind, ln_eps, s);
}

template <int FORM, bool XVEC>
hipError_t launch_pattern(const sbn_packed* h, const int8_t* xq, int64_t ld_q,
                          const float* absmax, int64_t T, void* y, int64_t ld_y, int out_kind,
                          hipStream_t s) {
  const Layout& L = h->L;
  if (T <= 16) return launch_gemv_int8(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);  // gemv_i8.hip
  const int64_t gx = (L.row_blocks + kGemmRowBlocks - 1) / kGemmRowBlocks;
  // 128-token tiles (CF = 8) when they number more than kSplitMaxTiles; otherwise 64-token tiles,
  // split over K as well if they are still that few. Same-process A/B, 2560 -> 6912 and
  // 6912 -> 2560 at T = 2048 and the 7B FFN shapes at T = 8192: 64-token tiles are 5-10% slower
  // where 128-token tiles fill the GPU, and 25% faster on 6912 -> 2560 (320 tiles, 52 us) than
  // 128-token tiles split over K (320 workgroups, 69 us: the halves' partial-sum exchange alone
  // cost 16 us).
  const bool wide = gx * ((T + 127) / 128) > kSplitMaxTiles;
  const int64_t gy = wide ? (T + 127) / 128 : (T + 63) / 64;
  // y offsets of the split-K handshake are 32-bit buffer offsets
  const bool y_fits = (double)T * (double)ld_y * 4.0 < 2147483647.0;
  const int ksplit = (gx * gy <= kSplitMaxTiles && L.quads >= 8 && y_fits) ? 2 : 1;
  // 512-row tiles (8 waves, one workgroup per CU) where they still number kWideMinTiles: the
  // activation tile of a K step then feeds twice the MFMAs (see the kernel's header).
  const int64_t gx8 = (L.row_blocks + 2 * kGemmRowBlocks - 1) / (2 * kGemmRowBlocks);
  const bool w8 = wide && gx8 * gy >= kWideMinTiles;
#define SBN_GEMM(CF, WW, GX)                                                                   \
  do {                                                                                         \
    hipError_t e = allow_smem(bitlinear_gemm<FORM, XVEC, CF, WW>, gemm_smem(CF));              \
    if (e != hipSuccess) return e;                                                             \
    hipLaunchKernelGGL((bitlinear_gemm<FORM, XVEC, CF, WW>), dim3((unsigned)(GX * gy * ksplit)), \
                       dim3(WW * 64), gemm_smem(CF), s, h->mask, h->codes, L,                   \
                       h->gamma_out(), xq, ld_q, absmax, T, y, ld_y, out_kind, (int)GX, (int)gy, \
                       ksplit, h->gemm_sync, h->splitk_spin_limit, h->splitk_publish);        \
  } while (0)
  if constexpr (XVEC && FORM != kFormKept) {  // positional bricks through a bounded resource
    // One round of 512-row tiles that fills at least kWideMinTiles of the CUs: the widest token
    // tile (128, 96 or 64 tokens) whose tile count lies in [kWideMinTiles, kOneRoundTiles].
    // Same-box A/B at T = 4096: 2560 -> 2560 38.8 -> 28.2 us and 6912 -> 2560 81.5 -> 60.4 us
    // with 96-token tiles (215 tiles) against 128-token tiles of 256 rows (320 tiles, two per CU
    // on 64 CUs); 2560 -> 6912 at T = 2048 keeps 128-token tiles (224). 48-token tiles (215 on
    // 6912 -> 2560 at T = 2048) ran in the time of the 320 64-token tiles of 256 rows there
    // (39.0 against 39.7 us) and fetched 16% more (58.3 against 50.4 MB), so they are not used.
    auto one_round = [&](int cf) {
      const int64_t tiles = gx8 * ((T + 16 * cf - 1) / (16 * cf));
      return tiles >= kWideMinTiles && tiles <= kOneRoundTiles;
    };
#define SBN_GEMM8(CF)                                                                          \
  do {                                                                                         \
    const int64_t gyc = (T + 16 * CF - 1) / (16 * CF);                                         \
    hipError_t e = allow_smem(bitlinear_gemm<FORM, XVEC, CF, 8>, gemm_smem(CF));               \
    if (e != hipSuccess) return e;                                                             \
    hipLaunchKernelGGL((bitlinear_gemm<FORM, XVEC, CF, 8>), dim3((unsigned)(gx8 * gyc)),        \
                       dim3(8 * 64), gemm_smem(CF), s, h->mask, h->codes, L, h->gamma_out(),    \
                       xq, ld_q, absmax, T, y, ld_y, out_kind, (int)gx8, (int)gyc, 1,           \
                       h->gemm_sync, h->splitk_spin_limit, h->splitk_publish);                 \
    return hipGetLastError();                                                                  \
  } while (0)
    if (one_round(8)) SBN_GEMM8(8);
    if (one_round(6)) SBN_GEMM8(6);
    if (one_round(4)) SBN_GEMM8(4);
#undef SBN_GEMM8
    if (w8) {
      SBN_GEMM(8, 8, gx8);
      return hipGetLastError();
    }
  }
  if (wide) {
    SBN_GEMM(8, 4, gx);
  } else {
    SBN_GEMM(4, 4, gx);
  }
#undef SBN_GEMM
  return hipGetLastError();
}

template <int FORM>
hipError_t launch_pattern_x(const sbn_packed* h, const int8_t* xq, int64_t ld_q,
                            const float* absmax, int64_t T, void* y, int64_t ld_y, int out_kind,
                            hipStream_t s) {
  const bool xvec = ((uintptr_t)xq % 16 == 0) && (ld_q % 16 == 0) && (h->L.K % 16 == 0) &&
                    ld_q < (int64_t{1} << 24);
  if (xvec) return launch_pattern<FORM, true>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
  return launch_pattern<FORM, false>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
}

template <int FORM, bool XVEC>
hipError_t launch_gemv_fused(const sbn_packed* h, const uint16_t* x, int64_t ld_x, int64_t T,
                             int8_t* xq, int64_t ld_q, float* absmax, void* y, int64_t ld_y,
                             int out_kind, float ln_eps, hipStream_t s) {
  return launch_gemv<FORM, true, XVEC>(h, x, ld_x, xq, ld_q, absmax, T, y, ld_y, out_kind, ln_eps,
                                       s);
}

// The one-token step with the k:256 outlier term in the same launch (bitlinear_gemv_outl).
template <int FORM>
hipError_t launch_gemv_outl(const sbn_packed* h, const uint16_t* x, int8_t* xq, int64_t ld_q,
                            float* absmax, float* y, hipStream_t s) {
  const Layout& L = h->L;
  const int W = (int)std::min<int64_t>(kGemvMaxWaves, (L.quads + kGemvMaxQ - 1) / kGemvMaxQ);
  const int Q = (int)((L.quads + W - 1) / W);
  const size_t smem = gemv_outl_smem(L.K, h->outlier_k);
#define SBN_GEMV_OUTL(QQ)                                                                      \
  do {                                                                                         \
    hipError_t e = allow_smem(bitlinear_gemv_outl<FORM, QQ>, smem);                            \
    if (e != hipSuccess) return e;                                                             \
    hipLaunchKernelGGL((bitlinear_gemv_outl<FORM, QQ>), dim3((unsigned)L.row_blocks),            \
                       dim3(64 * W), smem, s, h->mask, h->codes, L, h->gamma_out(), x, xq,       \
                       ld_q, absmax, y, h->opos, h->oval, h->outlier_k);                       \
  } while (0)
  if (Q == 1) {
    SBN_GEMV_OUTL(1);
  } else if (Q == 2) {
    SBN_GEMV_OUTL(2);
  } else {
    SBN_GEMV_OUTL(3);
  }
#undef SBN_GEMV_OUTL
  return hipGetLastError();
}

hipError_t launch_bitlinear_bf16_plain(const sbn_packed* h, const uint16_t* x, int64_t ld_x,
                                       int64_t T, int8_t* xq, int64_t ld_q, float* absmax,
                                       void* y, int64_t ld_y, int out_kind, float ln_eps,
                                       hipStream_t s);

}  // namespace

// The bf16-input forward, with the k:256 outlier term when the handle has one (fp32 output): in
// the same launch for one token (no LayerNorm, positional or structured codes, n_out a multiple of
// 16), otherwise by the outlier kernel after the forward.
hipError_t launch_bitlinear_bf16(const sbn_packed* h, const uint16_t* x, int64_t ld_x, int64_t T,
                                 int8_t* xq, int64_t ld_q, float* absmax, void* y, int64_t ld_y,
                                 int out_kind, float ln_eps, hipStream_t s) {
  const Layout& L = h->L;
  if (T == 0) return hipSuccess;
  const bool outl = h->outlier_k > 0 && out_kind == SBN_OUT_F32 && L.n_out > 0;
  if (outl && T == 1 && ln_eps <= 0.0f && !h->compact && L.n_out % 16 == 0 &&
      L.quads <= (int64_t)kGemvMaxWaves * kGemvMaxQ && (uintptr_t)x % 8 == 0 &&
      2.0 * (double)(L.K >> 8) * h->outlier_k * (double)L.n_out < 2147483647.0) {
    float* yf = static_cast<float*>(y);
    if (L.form == kFormSparse24) return launch_gemv_outl<kFormSparse24>(h, x, xq, ld_q, absmax, yf, s);
    if (L.form == kFormPositional)
      return launch_gemv_outl<kFormPositional>(h, x, xq, ld_q, absmax, yf, s);
    return launch_gemv_outl<kFormKept>(h, x, xq, ld_q, absmax, yf, s);
  }
  hipError_t e = launch_bitlinear_bf16_plain(h, x, ld_x, T, xq, ld_q, absmax, y, ld_y, out_kind,
                                             ln_eps, s);
  if (e == hipSuccess && outl)
    e = launch_outlier_add(h, xq, ld_q, absmax, T, static_cast<float*>(y), ld_y, s);
  return e;
}

namespace {

hipError_t launch_bitlinear_bf16_plain(const sbn_packed* h, const uint16_t* x, int64_t ld_x,
                                       int64_t T, int8_t* xq, int64_t ld_q, float* absmax,
                                       void* y, int64_t ld_y, int out_kind, float ln_eps,
                                       hipStream_t s) {
  const Layout& L = h->L;
  // one token, no LayerNorm: the entry with preloaded arguments (gemv_bf16.hip)
  if (gemv_bf16_one_fits(h, x, T, ln_eps))
    return launch_gemv_bf16_one(h, x, xq, ld_q, absmax, y, ld_y, out_kind, s);
  if (L.n_out > 0 && T <= kFusedMaxT && L.quads <= (int64_t)kGemvMaxWaves * kGemvMaxQ) {
    const bool xvec = ((uintptr_t)x % 8 == 0) && (ld_x % 4 == 0) && (L.K % 4 == 0);
#define SBN_FUSED(FF)                                                                          \
  return xvec ? launch_gemv_fused<FF, true>(h, x, ld_x, T, xq, ld_q, absmax, y, ld_y, out_kind,  \
                                            ln_eps, s)                                         \
              : launch_gemv_fused<FF, false>(h, x, ld_x, T, xq, ld_q, absmax, y, ld_y, out_kind, \
                                             ln_eps, s)
    if (h->compact) {
      return xvec ? launch_gemv_compact<true, true>(h, x, ld_x, xq, ld_q, absmax, T, y, ld_y,
                                                    out_kind, ln_eps, s)
                  : launch_gemv_compact<true, false>(h, x, ld_x, xq, ld_q, absmax, T, y, ld_y,
                                                     out_kind, ln_eps, s);
    }
    if (L.form == kFormSparse24) SBN_FUSED(kFormSparse24);
    if (L.form == kFormPositional) SBN_FUSED(kFormPositional);
    SBN_FUSED(kFormKept);
#undef SBN_FUSED
  }
  hipError_t e = ln_eps > 0.0f ? launch_ln_quantize_act(x, T, L.K, ld_x, ln_eps, xq, ld_q, absmax, s)
                               : launch_quantize_act(x, T, L.K, ld_x, xq, ld_q, absmax, s);
  if (e != hipSuccess) return e;
  return launch_bitlinear(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
}

}  // namespace

bool gemv_group_fused_fits(const sbn_packed* h0, const uint16_t* x, int64_t ld_x, int64_t T) {
  (void)x;
  (void)ld_x;
  return T <= kFusedMaxT && h0->L.quads <= (int64_t)kGemvMaxWaves * kGemvMaxQ;
}

hipError_t launch_gemv_group_bf16(const sbn_packed* const* hs, int count, const uint16_t* x,
                                  int64_t ld_x, int64_t T, int8_t* xq, int64_t ld_q,
                                  float* absmax, void* const* ys, const int64_t* ld_ys,
                                  int out_kind, float ln_eps, hipStream_t s) {
  GemvGroup G;
  const int blocks = make_group(hs, count, ys, ld_ys, G);
  const Layout& L = hs[0]->L;
  const bool xvec = ((uintptr_t)x % 8 == 0) && (ld_x % 4 == 0) && (L.K % 4 == 0);
#define SBN_GF(FF)                                                                             \
  return xvec ? launch_gemv_group_fused<FF, true>(G, blocks, L, x, ld_x, xq, ld_q, absmax, T,   \
                                                  out_kind, ln_eps, s)                         \
              : launch_gemv_group_fused<FF, false>(G, blocks, L, x, ld_x, xq, ld_q, absmax, T,  \
                                                   out_kind, ln_eps, s)
  if (L.form == kFormSparse24) SBN_GF(kFormSparse24);
  if (L.form == kFormPositional) SBN_GF(kFormPositional);
  SBN_GF(kFormKept);
#undef SBN_GF
}

hipError_t launch_bitlinear(const sbn_packed* h, const int8_t* xq, int64_t ld_q,
                            const float* absmax, int64_t T, void* y, int64_t ld_y, int out_kind,
                            hipStream_t s) {
  const Layout& L = h->L;
  if (L.n_out == 0 || T == 0) return hipSuccess;
  if (L.form == kFormSparse24)
    return launch_pattern_x<kFormSparse24>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
  if (L.form == kFormPositional)
    return launch_pattern_x<kFormPositional>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
  return launch_pattern_x<kFormKept>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
}

}  // namespace sbn
