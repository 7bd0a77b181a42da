// Entry of the int8-input GEMV (T <= 16; "Microsoft BitNet 1.58: The Era of 1-Bit Large Language
// Models", section "The BitLinear Layer", operations 4 and 5). The kernel body is the one the
// bf16-input kernels use (gemv.hpp); this file is compiled with kernel-argument preloading, and
// its entry takes the values its first loads need (code plane, activations, quad count, K, leading
// dimension, token count, wave count, a', gamma) as leading scalar arguments, so those loads go out without waiting
// for a scalar load of the argument block (3.77 -> 3.57 us at T = 1 and 5.64 -> 5.35 us at T = 16
// on the 2560 -> 6912 shape). The bf16-input kernels keep their own argument order: moving their
// arguments the same way made them slower.
#include <stdlib.h>

#include "gemv.hpp"

namespace sbn {
namespace {

template <int FORM, bool XVEC, int Q, bool XBUF>
__global__ __launch_bounds__(kGemvMaxWaves * 64) void bitlinear_gemv_i8(
    const uint8_t* __restrict__ code_plane, const void* __restrict__ xin, int nq, int K, int ld_x,
    int T, int W, const float* __restrict__ absmax, const float* __restrict__ gamma_p,
    const uint8_t* __restrict__ mask_plane, Layout L, void* __restrict__ y, int64_t ld_y,
    int out_kind) {
  gemv_body<FORM, false, XVEC, Q, false, XBUF>(mask_plane, code_plane, L, K, nq, W, gamma_p, xin,
                                               (int64_t)ld_x, nullptr, 0,
                                               const_cast<float*>(absmax), (int64_t)T, y, ld_y,
                                               out_kind, 0.0f, (int64_t)blockIdx.x, false);
}

// The grouped int8 GEMV (members as in bitlinear_gemv_group, gemv.hpp).
template <int FORM, bool XVEC, int Q, bool XBUF>
__global__ __launch_bounds__(kGemvMaxWaves * 64) void bitlinear_gemv_i8_group(
    const void* __restrict__ xin, int nq, int K, int ld_x, int T, int W,
    const float* __restrict__ absmax, GemvGroup G, Layout L, int out_kind) {
  int64_t rb;
  const int i = group_member(G, (int)blockIdx.x, rb);
  Layout Lm = L;
  Lm.n_out = G.m[i].n_out;
  gemv_body<FORM, false, XVEC, Q, false, XBUF>(G.m[i].mask, G.m[i].codes, Lm, K, nq, W,
                                               G.m[i].gamma, xin, (int64_t)ld_x, nullptr, 0,
                                               const_cast<float*>(absmax), (int64_t)T, G.m[i].y,
                                               G.m[i].ld_y, out_kind, 0.0f, rb, false);
}

// The int8 GEMV for K past one batch of the kernel above (more than 48 quads; e.g. 8192 x 28672,
// 112 quads): every wave issues the brick loads of all its quads at once (up to kDeepMaxQ, so one
// pass covers K <= 32768) instead of taking batches of three in turn, then streams its activation
// pieces two quads ahead of the products. Its loads return in order, so the activations of quad i
// are in once the bricks are; the products of quad i then overlap the activation loads of quads
// i + 1 and i + 2. Only the lanes of present tokens load activations (the others are masked
// off, so a one-token launch does not move 60 lanes' worth of empty pieces through the address
// units). Positional and 2:4 codes; rows of x_q 16-byte aligned, ld_q % 16 == 0, K % 16 == 0 (the
// launcher checks). Same-process A/B against the batched kernel (us): 8192 x 28672 at 8:16, one
// token 20.9 -> 18.2, sixteen 38.3 -> 34.5; 5120 x 13824 at 6:8, 11.0 -> 9.9 and 21.3 -> 18.7.
// (Without the masking the new kernel was slower at one token: 24.2 us.)
constexpr int kDeepMaxQ = 8;

// RB row blocks per workgroup share the activation loads (each wave's B operands serve RB sets of
// bricks): with 16 tokens the activation pieces outweigh the bricks, and RB = 2 halves them.
// The workgroup computes row blocks rb0 .. rb0 + RB - 1 of the weight whose code plane, scale and
// output are passed.
template <int FORM, int Q, int RB>
__device__ __forceinline__ void deep_body(
    const uint8_t* __restrict__ code_plane, const int8_t* __restrict__ xq, int nq, int K,
    int ld_q, int T, int W, const float* __restrict__ absmax, const float* __restrict__ gamma_p,
    void* __restrict__ y, int64_t ld_y, int64_t n_out, int out_kind, int cn, int csb,
    const int64_t rb0) {
  constexpr bool CMP = compact_form(FORM);
  static_assert(FORM == kFormPositional || FORM == kFormSparse24 || (CMP && RB == 1),
                "positional, 2:4 or (one row block) compact codes");
  __shared__ v4i red[RB][kGemvMaxWaves][64];
  __shared__ uint32_t clut[CMP ? 256 : 1];  // compact nibble table
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int t = lane & 15, g = lane >> 4;
  const bool tok_ok = t < T;
  // row blocks of this workgroup inside the stored (padded) plane: with RB = 3 the last
  // workgroup can reach past it, and its missing row blocks read zero
  const int64_t rb_pad = ((n_out + 15) / 16 + kPadRowBlocks - 1) / kPadRowBlocks * kPadRowBlocks;
  const int rb_in = (int)min<int64_t>(RB, rb_pad - rb0);
  // The RB row blocks' quads are consecutive in the plane; stored row blocks are padded to a
  // multiple of 16, so a last block past n_out exists (zero bricks; its rows are not stored).
  // Compact plane: a quad takes cq = 512 + 8 csb bytes (the lanes' nonzero masks, then their sign
  // slots as one bit stream); the range ends kCompactSlack bytes past the row block's last quad
  // (the plane has that slack), which covers every lane's three-word sign load.
  const int cq = CMP ? (int)compact_quad_bytes(csb) : 1024;
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(code_plane + rb0 * nq * cq), (short)0,
      rb_in * nq * cq + (CMP ? kCompactSlack : 0), kBufDword3);
  uint32_t codes[RB][Q][4];
  uint32_t cmask[CMP ? Q : 1][2];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int i = 0; i < Q; ++i) {
      const int q = wave + i * W;
      if constexpr (CMP) {
        // the lane's nonzero mask and the three words holding its csb sign bits; quads past the
        // last read zero (an offset past the range)
        const int qo = q < nq ? q * cq : nq * cq + kCompactSlack;
        const v2u mk = __builtin_amdgcn_raw_buffer_load_b64(crs, lane * 8, qo, kPlaneLoad);
        const int sbit = lane * csb;
        const v3u sg = __builtin_amdgcn_raw_buffer_load_b96(
            crs, kCompactMaskBytes + 4 * (sbit >> 5), qo, kPlaneLoad);
        cmask[i][0] = mk[0]; cmask[i][1] = mk[1];
        codes[r][i][0] = sg[0]; codes[r][i][1] = sg[1]; codes[r][i][2] = sg[2];
        codes[r][i][3] = (uint32_t)(sbit & 31);
      } else {
        const v4i c = __builtin_amdgcn_raw_buffer_load_b128(
            crs, lane * 16, q < nq ? (r * nq + q) * 1024 : RB * nq * 1024, kPlaneLoad);
        codes[r][i][0] = (uint32_t)c[0]; codes[r][i][1] = (uint32_t)c[1];
        codes[r][i][2] = (uint32_t)c[2]; codes[r][i][3] = (uint32_t)c[3];
      }
    }
  if constexpr (CMP) {
    for (int e = threadIdx.x; e < 256; e += blockDim.x) clut[e] = compact_nibble_entry(e);
    __syncthreads();  // the table, after the plane loads went out
  }
  // one resource over the T activation rows: quads past the last read zero (offsets past the
  // range); (T - 1) ld_q + K < 2^31 (T <= 16, ld_q <= 2^26)
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(xq), (short)0, (int)((int64_t)(T - 1) * ld_q + K), kBufDword3);
  auto load_x = [&](int i, v4i (&b)[4]) {
    const int q = wave + i * W;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int voff = q < nq ? t * ld_q + 16 * b_chunk<FORM>(g, j) : 0x7FFFFFF0;
      if (tok_ok) {
        b[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, voff, q < nq ? q * kQuadK : 0, 0);
      } else {
        b[j] = v4i{0, 0, 0, 0};
      }
    }
  };
  const float gamma = gamma_p[0];
  const float a_t = out_kind == SBN_OUT_F32 && tok_ok ? absmax[t] : 0.0f;
  v4i bx[3][4];
  load_x(0, bx[0]);
  if (Q > 1) load_x(1, bx[1]);
  v4i acc[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) acc[r] = v4i{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < Q; ++i) {
    if (i + 2 < Q) load_x(i + 2, bx[(i + 2) % 3]);
    v4i(&b)[4] = bx[i % 3];
    if (wave + i * W < nq) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if constexpr (FORM == kFormSparse24) {
#pragma unroll
          for (int blk = 0; blk < 2; ++blk) {
            uint32_t a[4];
            exp_word_to_i8(codes[r][i][2 * blk], a);
            acc[r] = smfmac16(a, b[2 * blk], b[2 * blk + 1], codes[r][i][2 * blk + 1], acc[r]);
          }
        } else if constexpr (CMP) {
          uint32_t a[16];
          const uint32_t sh = codes[r][i][3];
          const uint32_t lo = __builtin_amdgcn_alignbit(codes[r][i][1], codes[r][i][0], sh);
          const uint32_t hi = __builtin_amdgcn_alignbit(codes[r][i][2], codes[r][i][1], sh);
          decode_compact<compact_m(FORM)>(cmask[i], lo, hi, cn, csb, clut, a);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[r] = mfma16(a + 4 * j, b[j], acc[r]);
        } else {
          uint32_t a[16];
#pragma unroll
          for (int j = 0; j < 4; ++j) exp_word_to_i8(codes[r][i][j], a + 4 * j);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[r] = mfma16(a + 4 * j, b[j], acc[r]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RB; ++r) red[r][wave][lane] = acc[r];
  __syncthreads();
  // wave r sums row block r (wave 0 takes all of them when the workgroup has fewer waves)
  if (wave >= RB || !tok_ok) return;
  const float step = out_kind == SBN_OUT_F32 ? a_t / 127.0f : 0.0f;
  for (int r = wave; r < RB; r += W) {
    v4i sum = red[r][0][lane];
    for (int w = 1; w < W; ++w) sum += red[r][w][lane];
    const int64_t row0 = (rb0 + r) * 16 + 4 * g;
    const bool vec = ((uintptr_t)y % 16 == 0) && (ld_y % 4 == 0) && row0 + 3 < n_out;
    if (vec) {
      if (out_kind == SBN_OUT_I32_ACC) {
        *reinterpret_cast<v4i*>(reinterpret_cast<int32_t*>(y) + t * ld_y + row0) = sum;
      } else {
        float4 f;
        f.x = __fmul_rn(__fmul_rn((float)sum[0], gamma), step);
        f.y = __fmul_rn(__fmul_rn((float)sum[1], gamma), step);
        f.z = __fmul_rn(__fmul_rn((float)sum[2], gamma), step);
        f.w = __fmul_rn(__fmul_rn((float)sum[3], gamma), step);
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + t * ld_y + row0) = f;
      }
    } else {
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = row0 + i;
        if (row < n_out) store_out(y, ld_y, out_kind, t, row, sum[i], gamma, step);
      }
    }
  }
}

template <int FORM, int Q, int RB>
__global__ __launch_bounds__(kGemvMaxWaves * 64) void bitlinear_gemv_i8_deep(
    const uint8_t* __restrict__ code_plane, const int8_t* __restrict__ xq, int nq, int K,
    int ld_q, int T, int W, const float* __restrict__ absmax, const float* __restrict__ gamma_p,
    void* __restrict__ y, int64_t ld_y, int64_t n_out, int out_kind, int cn, int csb) {
  deep_body<FORM, Q, RB>(code_plane, xq, nq, K, ld_q, T, W, absmax, gamma_p, y, ld_y, n_out,
                         out_kind, cn, csb, (int64_t)blockIdx.x * RB);
}

// The grouped launch of the kernel above (members as in bitlinear_gemv_i8_group, their row blocks
// taken RB at a time: member i's workgroups are [rb_end[i-1], rb_end[i]), ceil(row blocks / RB)
// of them).
template <int FORM, int Q, int RB>
__global__ __launch_bounds__(kGemvMaxWaves * 64) void bitlinear_gemv_i8_deep_group(
    const int8_t* __restrict__ xq, int nq, int K, int ld_q, int T, int W,
    const float* __restrict__ absmax, GemvGroup G, int out_kind) {
  int64_t wg;
  const int i = group_member(G, (int)blockIdx.x, wg);
  deep_body<FORM, Q, RB>(G.m[i].codes, xq, nq, K, ld_q, T, W, absmax, G.m[i].gamma, G.m[i].y,
                         G.m[i].ld_y, G.m[i].n_out, out_kind, 0, 0, wg * RB);
}

// One to four tokens past one batch (49 to 128 quads): the workgroup first copies the activation
// rows into LDS (1 KB pieces, global -> LDS directly, issued before the brick loads so they come
// back first), and the waves read their B operands from there. The waves then keep no activation
// registers (64 or fewer VGPRs against about 100 in bitlinear_gemv_i8_deep), so two workgroups of
// 16 waves fit a CU and a launch of 512 row blocks runs in one round instead of two, and quad i is
// multiplied as soon as its bricks land. XC: LDS pieces per wave (the launcher's round-up of
// T * Kp / 1 KB / W); pieces past the rows go to a dummy KB past them. Same-box A/B against
// bitlinear_gemv_i8_deep at one token (us): 8192 x 28672 8:16 18.2 -> 13.9 (4.2 TB/s), 2:4
// 17.0 -> 13.1, 5120 x 13824 6:8 9.9 -> 7.5; the compact plane 23.0 -> 23.0 (8:16) and
// 13.1 -> 11.2 (6:8).
template <int FORM, int Q, int XC>
__global__ __launch_bounds__(kGemvMaxWaves * 64) void bitlinear_gemv_i8_deep_xl(
    const uint8_t* __restrict__ code_plane, const int8_t* __restrict__ xq, int nq, int K,
    int ld_q, int T, int W, const float* __restrict__ absmax, const float* __restrict__ gamma_p,
    void* __restrict__ y, int64_t ld_y, int64_t n_out, int out_kind, int cn, int csb) {
  constexpr bool CMP = compact_form(FORM);
  extern __shared__ __attribute__((aligned(16))) uint8_t xl_s[];  // T rows of Kp bytes, dummy KB
  __shared__ v4i red[kGemvMaxWaves][64];
  __shared__ uint32_t clut[CMP ? 256 : 1];  // compact nibble table
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int64_t rb0 = blockIdx.x;
  const int t = lane & 15, g = lane >> 4;
  const bool tok_ok = t < T;
  const int kc = (K + 1023) >> 10, Kp = kc << 10;  // 1 KB pieces per row, padded row length
  // Activation pieces: piece c = wave + i W is row c / kc, bytes (c % kc) KB .. +1 KB (past K:
  // zero, the resource ends with the row); pieces past the T rows read nothing and land in the
  // dummy KB at T Kp.
#pragma unroll
  for (int i = 0; i < XC; ++i) {
    const int c = wave + i * W;
    const bool real = c < T * kc;
    const int tt = real ? c / kc : 0, cc = real ? c % kc : 0;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(xq + (int64_t)tt * ld_q + cc * 1024), (short)0,
        real ? K - cc * 1024 : 0, kBufDword3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (lds_ptr)(xl_s + (real ? tt * Kp + cc * 1024 : T * Kp)), 16, lane * 16, 0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);  // the pieces go out before the bricks
  const int cq = CMP ? (int)compact_quad_bytes(csb) : 1024;
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(code_plane + rb0 * nq * cq), (short)0,
      nq * cq + (CMP ? kCompactSlack : 0), kBufDword3);
  uint32_t codes[Q][4];
  uint32_t cmask[CMP ? Q : 1][2];
#pragma unroll
  for (int i = 0; i < Q; ++i) {
    const int q = wave + i * W;
    if constexpr (CMP) {
      const int qo = q < nq ? q * cq : nq * cq + kCompactSlack;
      const v2u mk = __builtin_amdgcn_raw_buffer_load_b64(crs, lane * 8, qo, kPlaneLoad);
      const int sbit = lane * csb;
      const v3u sg = __builtin_amdgcn_raw_buffer_load_b96(
          crs, kCompactMaskBytes + 4 * (sbit >> 5), qo, kPlaneLoad);
      cmask[i][0] = mk[0]; cmask[i][1] = mk[1];
      codes[i][0] = sg[0]; codes[i][1] = sg[1]; codes[i][2] = sg[2];
      codes[i][3] = (uint32_t)(sbit & 31);
    } else {
      const v4i c = __builtin_amdgcn_raw_buffer_load_b128(crs, lane * 16,
                                                          q < nq ? q * 1024 : nq * 1024, kPlaneLoad);
      codes[i][0] = (uint32_t)c[0]; codes[i][1] = (uint32_t)c[1];
      codes[i][2] = (uint32_t)c[2]; codes[i][3] = (uint32_t)c[3];
    }
  }
  // The activation pieces went out first and return first: waiting until only the brick loads
  // (Q, or 2 Q for the compact plane) are in flight means this wave's pieces are in LDS.
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(CMP ? 2 * Q : Q));
  __builtin_amdgcn_sched_barrier(0);
  const float gamma = gamma_p[0];
  const float a_t = out_kind == SBN_OUT_F32 && tok_ok ? absmax[t] : 0.0f;
  if constexpr (CMP) {
    for (int e = threadIdx.x; e < 256; e += blockDim.x) clut[e] = compact_nibble_entry(e);
  }
  __syncthreads();  // every wave's pieces (and the nibble table)
  v4i acc = v4i{0, 0, 0, 0};
  const uint8_t* const xrow = xl_s + t * Kp;
#pragma unroll
  for (int i = 0; i < Q; ++i) {
    const int q = wave + i * W;
    if (q < nq) {
      v4i b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = tok_ok ? *reinterpret_cast<const v4i*>(xrow + q * kQuadK + 16 * b_chunk<FORM>(g, j))
                      : v4i{0, 0, 0, 0};
      if constexpr (FORM == kFormSparse24) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          uint32_t a[4];
          exp_word_to_i8(codes[i][2 * blk], a);
          acc = smfmac16(a, b[2 * blk], b[2 * blk + 1], codes[i][2 * blk + 1], acc);
        }
      } else if constexpr (CMP) {
        uint32_t a[16];
        const uint32_t sh = codes[i][3];
        const uint32_t lo = __builtin_amdgcn_alignbit(codes[i][1], codes[i][0], sh);
        const uint32_t hi = __builtin_amdgcn_alignbit(codes[i][2], codes[i][1], sh);
        decode_compact<compact_m(FORM)>(cmask[i], lo, hi, cn, csb, clut, a);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mfma16(a + 4 * j, b[j], acc);
      } else {
        uint32_t a[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) exp_word_to_i8(codes[i][j], a + 4 * j);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mfma16(a + 4 * j, b[j], acc);
      }
    }
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0 || !tok_ok) return;
  v4i sum = red[0][lane];
  for (int w = 1; w < W; ++w) sum += red[w][lane];
  const float step = out_kind == SBN_OUT_F32 ? a_t / 127.0f : 0.0f;
  const int64_t row0 = rb0 * 16 + 4 * g;
  const bool vec = ((uintptr_t)y % 16 == 0) && (ld_y % 4 == 0) && row0 + 3 < n_out;
  if (vec) {
    if (out_kind == SBN_OUT_I32_ACC) {
      *reinterpret_cast<v4i*>(reinterpret_cast<int32_t*>(y) + t * ld_y + row0) = sum;
    } else {
      float4 f;
      f.x = __fmul_rn(__fmul_rn((float)sum[0], gamma), step);
      f.y = __fmul_rn(__fmul_rn((float)sum[1], gamma), step);
      f.z = __fmul_rn(__fmul_rn((float)sum[2], gamma), step);
      f.w = __fmul_rn(__fmul_rn((float)sum[3], gamma), step);
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + t * ld_y + row0) = f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (row0 + i < n_out) store_out(y, ld_y, out_kind, t, row0 + i, sum[i], gamma, step);
  }
}

// Five to sixteen tokens past one batch (49 to 128 quads, positional or 2:4 codes): every row
// block of the kernels above re-reads all T activation rows (235 MB from L2 for 8192 x 28672 at
// T = 16, against 58.7 MB of codes). Here a workgroup takes 16 row blocks (256 rows, one per wave)
// and one K chunk of kKxQuads quads: the chunk's T x 1.75 KB of activations go to LDS once and serve
// all 16 waves, and the K chunks of a row group meet through int32 partial sums. At most 64 VGPRs,
// so two workgroups share a CU (8192 x 28672: 32 row groups x 16 chunks, one round). Same-box
// A/B at T = 16 against bitlinear_gemv_i8_deep (us): 8192 x 28672 8:16 34.8 -> 28.3, 2:4 33.2 ->
// 26.4, 5120 x 13824 6:8 18.8 -> 16.2 (8-quad chunks at 70 VGPRs, one workgroup per CU: 31.8,
// 31.9, 16.6). Each workgroup
// stores its waves' partial sums (16 KB) in the handle, waits for them, and counts its arrival on
// the row group's counter; the last arrival of the group (the C - 1-th after the others') adds
// the other chunks' partial sums to its own (integer sums: any order gives the same result),
// writes y and resets the counter. No workgroup waits for another. A row group's chunks run on one
// XCD (the grid is padded so that every XCD's contiguous run of the grouped order holds whole
// row groups; padding workgroups exit at once), so their partial sums and counter meet in that
// XCD's L2; the last arrival reads them past its L1.
template <int FORM, int XC>
__global__ __launch_bounds__(kGemvMaxWaves * 64) __attribute__((amdgpu_waves_per_eu(8, 8)))
void bitlinear_gemv_i8_kx(
    const uint8_t* __restrict__ code_plane, const int8_t* __restrict__ xq, int nq, int K,
    int ld_q, int T, const float* __restrict__ absmax, const float* __restrict__ gamma_p,
    void* __restrict__ y, int64_t ld_y, int64_t n_out, int out_kind, int C, int RG,
    uint8_t* __restrict__ part, uint32_t* __restrict__ count) {
  constexpr int KQ = kKxQuads;
  constexpr int kCk = KQ * kQuadK;  // activation bytes of one row in a chunk
  constexpr int kRow = 2048;        // their LDS row: two 1 KB pieces (KQ <= 8)
  static_assert(kCk <= kRow, "two pieces per row");
  __shared__ __attribute__((aligned(16))) uint8_t xs[17 * kRow];  // 16 rows, a dummy row
  __shared__ int last_s;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int lin = xcd_order((int)gridDim.x, (int)blockIdx.x);
  const int grp = lin / C, c = lin % C;
  if (grp >= RG) return;  // padding (the whole workgroup)
  const int64_t rb = (int64_t)grp * 16 + wave;
  const int t = lane & 15, g = lane >> 4;
  const bool tok_ok = t < T;
  // activation pieces: piece p = wave + i 16 of the chunk is row p / 2, bytes (p % 2) KB .. +1 KB
  // from the chunk's start (past K: zero; past the chunk: the next chunk's bytes, unused); pieces
  // past the T rows land in the dummy row
#pragma unroll
  for (int i = 0; i < XC; ++i) {
    const int pc = wave + i * kGemvMaxWaves;
    const bool real = pc < 2 * T;
    const int tt = real ? pc >> 1 : 0, hb = real ? pc & 1 : 0;
    const int64_t k0 = (int64_t)c * kCk + hb * 1024;
    const int64_t left = K - k0;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(xq + (int64_t)tt * ld_q + k0), (short)0,
        real && left > 0 ? (int)left : 0, kBufDword3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (lds_ptr)(xs + (real ? tt * kRow + hb * 1024 : 16 * kRow)), 16, lane * 16, 0, 0, 0);
  }
  // the token's a' with the pieces, so the last arrival's epilogue waits for no load of its own
  float a_t = 0.0f;
  if (out_kind == SBN_OUT_F32) a_t = absmax[tok_ok ? t : 0];
  __builtin_amdgcn_sched_barrier(0);  // the pieces go out before the bricks
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(code_plane + rb * nq * 1024), (short)0, nq * 1024, kBufDword3);
  uint32_t codes[KQ][4];
#pragma unroll
  for (int i = 0; i < KQ; ++i) {
    const int q = c * KQ + i;
    const v4i v = __builtin_amdgcn_raw_buffer_load_b128(crs, lane * 16,
                                                        q < nq ? q * 1024 : nq * 1024, kPlaneLoad);
    codes[i][0] = (uint32_t)v[0]; codes[i][1] = (uint32_t)v[1];
    codes[i][2] = (uint32_t)v[2]; codes[i][3] = (uint32_t)v[3];
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(KQ));  // only the brick loads are still in flight
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();  // every wave's pieces are in LDS
  v4i acc = v4i{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < KQ; ++i) {
    v4i b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = tok_ok ? *reinterpret_cast<const v4i*>(xs + t * kRow + i * kQuadK +
                                                    16 * b_chunk<FORM>(g, j))
                    : v4i{0, 0, 0, 0};
    if constexpr (FORM == kFormSparse24) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        uint32_t a[4];
        exp_word_to_i8(codes[i][2 * blk], a);
        acc = smfmac16(a, b[2 * blk], b[2 * blk + 1], codes[i][2 * blk + 1], acc);
      }
    } else {
      uint32_t a[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) exp_word_to_i8(codes[i][j], a + 4 * j);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mfma16(a + 4 * j, b[j], acc);
    }
  }
  // this chunk's partial sums: 16 waves x 64 lanes x 16 bytes at (group, chunk)
  uint8_t* const pg = part + (int64_t)grp * C * 16384;
  *reinterpret_cast<v4i*>(pg + c * 16384 + wave * 1024 + lane * 16) = acc;
  __builtin_amdgcn_s_waitcnt(0);  // the partial sums have reached L2
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(count + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_s = old == (uint32_t)(C - 1);
  }
  __syncthreads();
  if (!last_s) return;
  constexpr int kGlc = 1;  // buffer cache-policy bit sc0: read past L1
  const __amdgpu_buffer_rsrc_t pr =
      __builtin_amdgcn_make_buffer_rsrc(pg, (short)0, C * 16384, kBufDword3);
  const float gamma = gamma_p[0];
  // The other chunks' partial sums, kPB loads in flight per wait (their own chunk and chunks past
  // C take an offset past the range and read zero). One wait per load made the last arrival's
  // C - 1 L2 round trips serial.
  constexpr int kPB = 8;
  for (int c0 = 0; c0 < C; c0 += kPB) {
    v4i pv[kPB];
#pragma unroll
    for (int u = 0; u < kPB; ++u) {
      const int cc = c0 + u;
      pv[u] = __builtin_amdgcn_raw_buffer_load_b128(pr, wave * 1024 + lane * 16,
                                                    cc < C && cc != c ? cc * 16384 : C * 16384,
                                                    kGlc);
    }
#pragma unroll
    for (int u = 0; u < kPB; ++u) acc += pv[u];
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(count + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!tok_ok) return;
  const float step = out_kind == SBN_OUT_F32 ? a_t / 127.0f : 0.0f;
  const int64_t row0 = rb * 16 + 4 * g;
  const bool vec = ((uintptr_t)y % 16 == 0) && (ld_y % 4 == 0) && row0 + 3 < n_out;
  if (vec) {
    if (out_kind == SBN_OUT_I32_ACC) {
      *reinterpret_cast<v4i*>(reinterpret_cast<int32_t*>(y) + t * ld_y + row0) = acc;
    } else {
      float4 f;
      f.x = __fmul_rn(__fmul_rn((float)acc[0], gamma), step);
      f.y = __fmul_rn(__fmul_rn((float)acc[1], gamma), step);
      f.z = __fmul_rn(__fmul_rn((float)acc[2], gamma), step);
      f.w = __fmul_rn(__fmul_rn((float)acc[3], gamma), step);
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + t * ld_y + row0) = f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (row0 + i < n_out) store_out(y, ld_y, out_kind, t, row0 + i, acc[i], gamma, step);
  }
}

template <int FORM>
hipError_t launch_i8_kx(const sbn_packed* h, const int8_t* xq, int64_t ld_q, const float* absmax,
                        int64_t T, void* y, int64_t ld_y, int out_kind, hipStream_t s) {
  const Layout& L = h->L;
  const int C = h->kx_chunks;
  const int64_t RG = (L.row_blocks + 15) / 16, RGp = kx_row_groups(L.row_blocks);
  const unsigned blocks = (unsigned)(RGp * C);
  // activation pieces per wave: 2 T over 16 waves
  if (T <= 8) {
    hipLaunchKernelGGL((bitlinear_gemv_i8_kx<FORM, 1>), dim3(blocks), dim3(64 * kGemvMaxWaves), 0,
                       s, h->codes, xq, (int)L.quads, (int)L.K, (int)ld_q, (int)T, absmax,
                       h->gamma_out(), y, ld_y, L.n_out, out_kind, C, (int)RG, h->kx_part,
                       h->kx_count);
  } else {
    hipLaunchKernelGGL((bitlinear_gemv_i8_kx<FORM, 2>), dim3(blocks), dim3(64 * kGemvMaxWaves), 0,
                       s, h->codes, xq, (int)L.quads, (int)L.K, (int)ld_q, (int)T, absmax,
                       h->gamma_out(), y, ld_y, L.n_out, out_kind, C, (int)RG, h->kx_part,
                       h->kx_count);
  }
  return hipGetLastError();
}

template <int FORM>
hipError_t launch_i8_deep_xl(const sbn_packed* h, const int8_t* xq, int64_t ld_q,
                             const float* absmax, int64_t T, void* y, int64_t ld_y,
                             int out_kind, hipStream_t s) {
  const Layout& L = h->L;
  const int W = (int)std::min<int64_t>(kGemvMaxWaves, L.quads);
  const int Q = (int)((L.quads + W - 1) / W);
  const int64_t kc = (L.K + 1023) >> 10;
  const int64_t pieces = (T * kc + W - 1) / W;  // per wave
  const size_t smem = (size_t)(T * kc + 1) * 1024;
  const uint8_t* plane = compact_form(FORM) ? h->cplane : h->codes;
#define SBN_XL(QQ, XX)                                                                         \
  do {                                                                                         \
    hipError_t e = allow_smem(bitlinear_gemv_i8_deep_xl<FORM, QQ, XX>, smem);                  \
    if (e != hipSuccess) return e;                                                             \
    hipLaunchKernelGGL((bitlinear_gemv_i8_deep_xl<FORM, QQ, XX>), dim3((unsigned)L.row_blocks), \
                       dim3(64 * W), smem, s, plane, xq, (int)L.quads, (int)L.K, (int)ld_q,      \
                       (int)T, W, absmax, h->gamma_out(), y, ld_y, L.n_out, out_kind, L.n,      \
                       L.csb);                                                                 \
  } while (0)
#define SBN_XL_Q(XX)                                                                           \
  switch (Q) {                                                                                 \
    case 4: SBN_XL(4, XX); break;                                                              \
    case 5: SBN_XL(5, XX); break;                                                              \
    case 6: SBN_XL(6, XX); break;                                                              \
    case 7: SBN_XL(7, XX); break;                                                              \
    default: SBN_XL(8, XX); break;                                                             \
  }
  if (pieces <= 2) {
    SBN_XL_Q(2);
  } else if (pieces <= 4) {
    SBN_XL_Q(4);
  } else {
    SBN_XL_Q(8);
  }
#undef SBN_XL_Q
#undef SBN_XL
  return hipGetLastError();
}

template <int FORM, int RB>
hipError_t launch_i8_deep(const sbn_packed* h, const int8_t* xq, int64_t ld_q,
                          const float* absmax, int64_t T, void* y, int64_t ld_y, int out_kind,
                          hipStream_t s) {
  const Layout& L = h->L;
  const int W = (int)std::min<int64_t>(kGemvMaxWaves, L.quads);
  const int Q = (int)((L.quads + W - 1) / W);
  const unsigned blocks = (unsigned)((L.row_blocks + RB - 1) / RB);
  const uint8_t* plane = compact_form(FORM) ? h->cplane : h->codes;
#define SBN_DEEP(QQ)                                                                           \
  hipLaunchKernelGGL((bitlinear_gemv_i8_deep<FORM, QQ, RB>), dim3(blocks), dim3(64 * W), 0, s, \
                     plane, xq, (int)L.quads, (int)L.K, (int)ld_q, (int)T, W, absmax,            \
                     h->gamma_out(), y, ld_y, L.n_out, out_kind, L.n, L.csb)
  if constexpr (RB > 1) {  // (launched for one batch only: Q <= kGemvMaxQ)
    switch (Q) {
      case 1: SBN_DEEP(1); break;
      case 2: SBN_DEEP(2); break;
      default: SBN_DEEP(3); break;
    }
  } else {
    switch (Q) {
      case 1: SBN_DEEP(1); break;
      case 2: SBN_DEEP(2); break;
      case 3: SBN_DEEP(3); break;
      case 4: SBN_DEEP(4); break;
      case 5: SBN_DEEP(5); break;
      case 6: SBN_DEEP(6); break;
      case 7: SBN_DEEP(7); break;
      default: SBN_DEEP(8); break;
    }
  }
#undef SBN_DEEP
  return hipGetLastError();
}

// The one-token int8 GEMV with the k:256 outlier term in the same launch (fp32 output; planes
// [G k][n_out]); the term's arithmetic is that of the separate outlier kernel (gemv.hpp, OUTL).
template <int FORM, int Q>
__global__ __launch_bounds__(kGemvMaxWaves * 64) void bitlinear_gemv_i8_outl(
    const uint8_t* __restrict__ code_plane, const void* __restrict__ xin, int nq, int K, int W,
    const float* __restrict__ absmax, const float* __restrict__ gamma_p,
    const uint8_t* __restrict__ mask_plane, Layout L, void* __restrict__ y,
    const uint8_t* __restrict__ opos, const uint16_t* __restrict__ oval, int KO) {
  gemv_body<FORM, false, true, Q, false, true, true>(
      mask_plane, code_plane, L, K, nq, W, gamma_p, xin, (int64_t)K, nullptr, 0,
      const_cast<float*>(absmax), 1, y, (int64_t)L.n_out, SBN_OUT_F32, 0.0f, (int64_t)blockIdx.x,
      false, opos, oval, KO);
}

template <int FORM>
hipError_t launch_i8_outl(const sbn_packed* h, const int8_t* xq, const float* absmax, float* y,
                          hipStream_t s) {
  const Layout& L = h->L;
  const int W = (int)std::min<int64_t>(kGemvMaxWaves, L.quads);
  const int Q = (int)std::min<int64_t>(kGemvMaxQ, (L.quads + W - 1) / W);
  const size_t smem = gemv_outl_smem(L.K, h->outlier_k);
#define SBN_I8_OUTL(QQ)                                                                        \
  do {                                                                                         \
    hipError_t e = allow_smem(bitlinear_gemv_i8_outl<FORM, QQ>, smem);                         \
    if (e != hipSuccess) return e;                                                             \
    hipLaunchKernelGGL((bitlinear_gemv_i8_outl<FORM, QQ>), dim3((unsigned)L.row_blocks),         \
                       dim3(64 * W), smem, s, h->codes, static_cast<const void*>(xq),          \
                       (int)L.quads, (int)L.K, W, absmax, h->gamma_out(), h->mask, L,           \
                       static_cast<void*>(y), h->opos, h->oval, h->outlier_k);                  \
  } while (0)
  if (Q == 1) {
    SBN_I8_OUTL(1);
  } else if (Q == 2) {
    SBN_I8_OUTL(2);
  } else {
    SBN_I8_OUTL(3);
  }
#undef SBN_I8_OUTL
  return hipGetLastError();
}

// W waves (min(16, quads); for T > 4 see below) of Q = min(3, ceil(quads / W)) quads; past W Q
// quads the waves take batches of W Q in turn. Buffer-resource loads (XBUF) for T <= 4, and for
// up to 16 tokens when the launch is one batch; same-process A/B with non-temporal brick loads, T = 8 / 16 (us):
//   6912 x 2560   XBUF 3.95 / 5.0   branchy 4.37 / 5.7
//   2560 x 6912   XBUF 5.1  / 6.4   branchy 5.6  / 6.8
//   4096 x 11008  XBUF 6.9  / 9.2   branchy 7.5  / 9.7
//   5120 x 13824  XBUF 16.3 / 24.2  branchy 15.3 / 21.2   (two batches)
//   8192 x 28672  XBUF 25.9 / 40.0  branchy 26.2 / 37.9   (three batches)
// T > 4: the fewest quads per wave that fit (at most three), then the fewest waves at that
// count, so that few wave slots go empty. Same-process A/B at T = 8 / 16: 2560 x 6912 (27 quads;
// 14 waves of two instead of 16) 5.06 / 6.39 -> 4.78 / 5.96 us; 4096 x 11008 (43 quads; 15 waves
// of three instead of 16) 6.81 / 9.19 -> 6.64 / 8.87 us; unchanged for 10 quads and for batches.
void i8_shape(const Layout& L, int64_t T, int& W, int& Q, bool& xbuf) {
  W = (int)std::min<int64_t>(kGemvMaxWaves, L.quads);
  if (T > kFusedMaxT) {
    const int64_t q = std::min<int64_t>(kGemvMaxQ, (L.quads + kGemvMaxWaves - 1) / kGemvMaxWaves);
    W = (int)std::min<int64_t>(kGemvMaxWaves, (L.quads + q - 1) / q);
  }
  Q = (int)std::min<int64_t>(kGemvMaxQ, (L.quads + W - 1) / W);
  xbuf = T <= kFusedMaxT || L.quads <= (int64_t)kGemvMaxWaves * kGemvMaxQ;
}

template <int FORM, bool XVEC>
hipError_t launch_i8(const sbn_packed* h, const int8_t* xq, int64_t ld_q, const float* absmax,
                     int64_t T, void* y, int64_t ld_y, int out_kind, hipStream_t s) {
  const Layout& L = h->L;
  int W, Q;
  bool xbuf;
  i8_shape(L, T, W, Q, xbuf);
  const uint8_t* plane = compact_form(FORM) ? h->cplane : h->codes;
#define SBN_I8(QQ, XB)                                                                         \
  hipLaunchKernelGGL((bitlinear_gemv_i8<FORM, XVEC, QQ, XB>), dim3((unsigned)L.row_blocks),     \
                     dim3(64 * W), 0, s, plane, static_cast<const void*>(xq), (int)L.quads,      \
                     (int)L.K, (int)ld_q, (int)T, W, absmax, h->gamma_out(), h->mask, L, y,      \
                     ld_y, out_kind)
#define SBN_I8_Q(QQ)                                                                           \
  do {                                                                                         \
    if (xbuf) SBN_I8(QQ, true); else SBN_I8(QQ, false);                                        \
  } while (0)
  if (Q == 1) {
    SBN_I8_Q(1);
  } else if (Q == 2) {
    SBN_I8_Q(2);
  } else {
    SBN_I8_Q(3);
  }
#undef SBN_I8_Q
#undef SBN_I8
  return hipGetLastError();
}

template <bool XVEC>
hipError_t launch_i8_form(const sbn_packed* h, const int8_t* xq, int64_t ld_q,
                          const float* absmax, int64_t T, void* y, int64_t ld_y, int out_kind,
                          hipStream_t s) {
  const Layout& L = h->L;
  if (h->compact) {
    if (L.m == 4) return launch_i8<kFormCompact4, XVEC>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
    if (L.m == 8) return launch_i8<kFormCompact8, XVEC>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
    return launch_i8<kFormCompact16, XVEC>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
  }
  if (L.form == kFormSparse24)
    return launch_i8<kFormSparse24, XVEC>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
  if (L.form == kFormPositional)
    return launch_i8<kFormPositional, XVEC>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
  return launch_i8<kFormKept, XVEC>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
}

template <int FORM, bool XVEC>
hipError_t launch_i8_group(const GemvGroup& G, int blocks, const Layout& L, const int8_t* xq,
                           int64_t ld_q, const float* absmax, int64_t T, int out_kind,
                           hipStream_t s) {
  int W, Q;
  bool xbuf;
  i8_shape(L, T, W, Q, xbuf);
#define SBN_I8G(QQ, XB)                                                                        \
  hipLaunchKernelGGL((bitlinear_gemv_i8_group<FORM, XVEC, QQ, XB>), dim3((unsigned)blocks),     \
                     dim3(64 * W), 0, s, static_cast<const void*>(xq), (int)L.quads, (int)L.K,   \
                     (int)ld_q, (int)T, W, absmax, G, L, out_kind)
#define SBN_I8G_Q(QQ)                                                                          \
  do {                                                                                         \
    if (xbuf) SBN_I8G(QQ, true); else SBN_I8G(QQ, false);                                      \
  } while (0)
  if (Q == 1) {
    SBN_I8G_Q(1);
  } else if (Q == 2) {
    SBN_I8G_Q(2);
  } else {
    SBN_I8G_Q(3);
  }
#undef SBN_I8G_Q
#undef SBN_I8G
  return hipGetLastError();
}

template <bool XVEC>
hipError_t launch_i8_group_form(const GemvGroup& G, int blocks, const Layout& L,
                                const int8_t* xq, int64_t ld_q, const float* absmax, int64_t T,
                                int out_kind, hipStream_t s) {
  if (L.form == kFormSparse24)
    return launch_i8_group<kFormSparse24, XVEC>(G, blocks, L, xq, ld_q, absmax, T, out_kind, s);
  if (L.form == kFormPositional)
    return launch_i8_group<kFormPositional, XVEC>(G, blocks, L, xq, ld_q, absmax, T, out_kind, s);
  return launch_i8_group<kFormKept, XVEC>(G, blocks, L, xq, ld_q, absmax, T, out_kind, s);
}

}  // namespace

hipError_t launch_gemv_int8_group(const sbn_packed* const* hs, int count, const int8_t* xq,
                                  int64_t ld_q, const float* absmax, int64_t T, void* const* ys,
                                  const int64_t* ld_ys, int out_kind, hipStream_t s) {
  GemvGroup G;
  const Layout& L = hs[0]->L;
  const bool xvec = ((uintptr_t)xq % 16 == 0) && (ld_q % 16 == 0) && (L.K % 16 == 0);
  // More than four tokens, at most 16 quads, many row blocks in all: the kernel that shares each
  // wave's activation pieces among two (three from 640 row blocks on) row blocks of a member, as
  // for one weight.
  int64_t rbs = 0;
  bool compact = false;
  for (int i = 0; i < count; ++i) {
    rbs += hs[i]->L.row_blocks;
    compact = compact || hs[i]->compact;
  }
  if (xvec && T > kFusedMaxT && !compact && L.quads <= kGemvMaxWaves && rbs >= 320 &&
      (L.form == kFormPositional || L.form == kFormSparse24)) {
    const int W = (int)std::min<int64_t>(kGemvMaxWaves, L.quads);
#define SBN_DG(FF, RB)                                                                          \
  do {                                                                                          \
    const int blocks = make_group(hs, count, ys, ld_ys, G, RB);                                \
    hipLaunchKernelGGL((bitlinear_gemv_i8_deep_group<FF, 1, RB>), dim3((unsigned)blocks),          \
                       dim3(64 * W), 0, s, xq, (int)L.quads, (int)L.K, (int)ld_q, (int)T, W,     \
                       absmax, G, out_kind);                                                    \
    return hipGetLastError();                                                                   \
  } while (0)
    if (L.form == kFormSparse24) {
      if (rbs >= 640) SBN_DG(kFormSparse24, 3); else SBN_DG(kFormSparse24, 2);
    }
    if (rbs >= 640) SBN_DG(kFormPositional, 3); else SBN_DG(kFormPositional, 2);
#undef SBN_DG
  }
  const int blocks = make_group(hs, count, ys, ld_ys, G);
  if (xvec) return launch_i8_group_form<true>(G, blocks, L, xq, ld_q, absmax, T, out_kind, s);
  return launch_i8_group_form<false>(G, blocks, L, xq, ld_q, absmax, T, out_kind, s);
}

bool gemv_int8_outl_fits(const sbn_packed* h, const int8_t* xq, int64_t T) {
  const Layout& L = h->L;
  return h->outlier_k > 0 && T == 1 && !h->compact && L.n_out > 0 && L.n_out % 16 == 0 &&
         L.quads <= (int64_t)kGemvMaxWaves * kGemvMaxQ && (uintptr_t)xq % 16 == 0 &&
         L.K % 16 == 0 && 2.0 * (double)(L.K >> 8) * h->outlier_k * (double)L.n_out < 2147483647.0;
}

hipError_t launch_gemv_int8_outl(const sbn_packed* h, const int8_t* xq, const float* absmax,
                                 float* y, hipStream_t s) {
  if (h->L.form == kFormSparse24) return launch_i8_outl<kFormSparse24>(h, xq, absmax, y, s);
  if (h->L.form == kFormPositional) return launch_i8_outl<kFormPositional>(h, xq, absmax, y, s);
  return launch_i8_outl<kFormKept>(h, xq, absmax, y, s);
}

hipError_t launch_gemv_int8(const sbn_packed* h, const int8_t* xq, int64_t ld_q,
                            const float* absmax, int64_t T, void* y, int64_t ld_y, int out_kind,
                            hipStream_t s) {
  const bool xvec = ((uintptr_t)xq % 16 == 0) && (ld_q % 16 == 0) && (h->L.K % 16 == 0);
  const Layout& L = h->L;
  const bool deep_form = xvec && !h->compact &&
                         (L.form == kFormSparse24 || L.form == kFormPositional) &&
                         L.quads <= (int64_t)kGemvMaxWaves * kDeepMaxQ;
  // One to four tokens past one batch: activations staged in LDS (any code form but the kept one)
  if (xvec && T <= kFusedMaxT && L.quads > (int64_t)kGemvMaxWaves * kGemvMaxQ &&
      L.quads <= (int64_t)kGemvMaxWaves * kDeepMaxQ && L.form != kFormKept) {
    if (h->compact) {
      if (L.m == 4) return launch_i8_deep_xl<kFormCompact4>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
      if (L.m == 8) return launch_i8_deep_xl<kFormCompact8>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
      return launch_i8_deep_xl<kFormCompact16>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
    }
    if (L.form == kFormSparse24)
      return launch_i8_deep_xl<kFormSparse24>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
    return launch_i8_deep_xl<kFormPositional>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
  }
  // Five to sixteen tokens past one batch: split over K, activations shared through LDS
  if (xvec && T > kFusedMaxT && !h->compact && h->kx_chunks > 0 && L.quads >= kKxMinQuads &&
      L.quads <= kKxMaxQuads && (L.form == kFormPositional || L.form == kFormSparse24)) {
    if (L.form == kFormSparse24)
      return launch_i8_kx<kFormSparse24>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
    return launch_i8_kx<kFormPositional>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
  }
  // The compact plane past one batch takes the same kernel (one row block per workgroup).
  if (xvec && h->compact && L.quads > (int64_t)kGemvMaxWaves * kGemvMaxQ &&
      L.quads <= (int64_t)kGemvMaxWaves * kDeepMaxQ) {
    if (L.m == 4) return launch_i8_deep<kFormCompact4, 1>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
    if (L.m == 8) return launch_i8_deep<kFormCompact8, 1>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
    return launch_i8_deep<kFormCompact16, 1>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
  }
  if (deep_form && L.quads > (int64_t)kGemvMaxWaves * kGemvMaxQ) {
    if (L.form == kFormSparse24)
      return launch_i8_deep<kFormSparse24, 1>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
    return launch_i8_deep<kFormPositional, 1>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
  }
  // More than four tokens, one quad per wave and many row blocks: two row blocks per workgroup,
  // three from 640 row blocks on (about 220-230 workgroups either way). Same-process A/B against
  // the kernel above (us, T = 8 / 16): 6912 x 2560 3.96 / 4.98 -> 3.68 / 4.22, 11008 x 4096
  // 7.09 / 8.88 -> 5.83 / 7.18; slower with two or three quads per wave (2560 x 6912 4.81 / 6.10
  // -> 5.69 / 6.93) or few row blocks (2560 x 2560 3.12 / 3.52 -> 3.25 / 3.68). Three row blocks
  // against two: 11008 x 4096 6.05 / 7.70 -> 5.39 / 6.20, 6912 x 2560 3.73 / 4.26 -> 3.97 / 4.48
  // (four: 5.75 / 6.40 and 4.27 / 4.77).
  if (deep_form && T > kFusedMaxT && L.quads <= kGemvMaxWaves && L.row_blocks >= 320) {
    if (L.row_blocks >= 640) {
      if (L.form == kFormSparse24)
        return launch_i8_deep<kFormSparse24, 3>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
      return launch_i8_deep<kFormPositional, 3>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
    }
    if (L.form == kFormSparse24)
      return launch_i8_deep<kFormSparse24, 2>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
    return launch_i8_deep<kFormPositional, 2>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
  }
  if (xvec) return launch_i8_form<true>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
  return launch_i8_form<false>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
}

}  // namespace sbn
