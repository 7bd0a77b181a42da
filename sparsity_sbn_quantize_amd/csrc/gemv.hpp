// Device code of the n:m-sparse ternary x INT8 GEMV and the helpers it shares with the GEMM;
// included by bitlinear.hip (GEMM, bf16-input GEMV) and gemv_i8.hip (int8-input GEMV entry).
//
// "Microsoft BitNet 1.58: The Era of 1-Bit Large Language Models", section "The BitLinear
// Layer", operations 4 and 5; section "bitnet.cpp: Matrix-Free Inference".
#pragma once

#include <algorithm>

#include "sbn_internal.hpp"

namespace sbn {
namespace {


typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v4i mfma16(const uint32_t* a, v4i b, v4i c) {
  const v4i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3]};
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b, c, 0, 0, 0);
}

// Structured-sparse 2:4 MFMA over a 128-K block: a = the lane's 16 kept int8 weights, b = its 32
// dense activation bytes (K chunks g and g + 4 of the block, g = lane / 16), idx = the kept
// positions (2 bits per slot).
__device__ __forceinline__ v4i smfmac16(const uint32_t* a, v4i b_lo, v4i b_hi, uint32_t idx,
                                        v4i c) {
  const v4i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3]};
  const v8i bv = {b_lo[0], b_lo[1], b_lo[2], b_lo[3], b_hi[0], b_hi[1], b_hi[2], b_hi[3]};
  return __builtin_amdgcn_smfmac_i32_16x16x128_i8(av, bv, c, (int)idx, 0, 0);
}

// K chunk (16 bytes) of a 256-K quad that lane group g supplies as B operand piece j: slice j of
// brick g for the dense MFMA (chunk 4g + j); for the sparse form, chunks g and g + 4 of block 0,
// then of block 1 (chunk g + 4j).
template <int FORM>
__device__ __forceinline__ int b_chunk(int g, int j) {
  return FORM == kFormSparse24 ? g + 4 * j : 4 * g + j;
}

// Loads one brick: positional codes (16 bytes), or the kept form's mask (8 bytes) and code bytes.
template <int FORM>
__device__ __forceinline__ void load_brick(const Layout& L, const uint8_t* __restrict__ mask_plane,
                                           const uint8_t* __restrict__ code_plane, int64_t slot,
                                           uint32_t mask[2], uint32_t codes[4]) {
  mask[0] = mask[1] = 0;
  codes[0] = codes[1] = codes[2] = codes[3] = 0;
  if constexpr (FORM != kFormKept) {
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

template <int FORM>
__device__ __forceinline__ void decode(const Layout& L, const uint32_t mask[2],
                                       const uint32_t codes[4], uint32_t out[16]) {
  if constexpr (FORM == kFormPositional) {
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

__device__ __forceinline__ void store_out(void* y, int64_t ld_y, int out_kind, int64_t t,
                                          int64_t r, int acc, float gamma, float step) {
  if (out_kind == SBN_OUT_I32_ACC) {
    reinterpret_cast<int32_t*>(y)[t * ld_y + r] = acc;
  } else {
    const float v = __fmul_rn(__fmul_rn((float)acc, gamma), step);
    reinterpret_cast<float*>(y)[t * ld_y + r] = v;
  }
}

// GEMV (T <= 16): one workgroup per 16-row fragment row with W waves (set by the launcher); wave
// w takes the 256-K quads w, w + W, ... (at most kGemvMaxQ per batch; with int8 input, further
// batches of W * kGemvMaxQ quads follow for larger K). Every wave first issues its brick
// loads (HBM) and its activation loads (L2: every workgroup reads the same rows) straight into
// MFMA operand registers, then decodes and multiplies; the partial sums of the waves are combined
// through LDS once. Lane (t, g) supplies token t's 64 activation bytes at K offset 64g of each
// quad, matching the K slices of the bricks.
// FUSED (T <= 4): the activations are bf16. Every workgroup then computes the per-token absmax
// over K itself (lane maxima, then wave maxima combined through LDS) and quantizes the pieces it
// needs with the arithmetic of the quantize kernel, so the decode step is one launch with no int8
// copy of the activations between two kernels; workgroup 0 also writes x_q and a' for the caller.
// (For more tokens every workgroup would redo a quantization pass over all T x K activations;
// there the quantize kernel followed by the GEMV is faster.)
constexpr int kGemvMaxWaves = 16;
// Quads per wave in one batch (template Q <= 3, so the operands fit in registers): one batch
// covers K <= 16 * 3 * 256 = 12288; the int8-input GEMV runs ceil(quads / (3 W)) batches past that,
// the one-kernel bf16 path stays at one batch.
constexpr int kGemvMaxQ = 3;
constexpr int kFusedMaxT = 4;  // tokens of the one-kernel quantize-and-multiply path
// Cache policy of the brick loads (read once per call): nt. Same-process A/B on the 2560 -> 6912
// decode shape, against the default policy: one-kernel step 4.49 -> 4.16 us, with the LayerNorm
// 6.58 -> 5.82 us, the int8 GEMV unchanged (3.34 us); sc1 alone changed nothing. The outlier
// planes keep the default policy: nt there made the one-token outlier step slower (8.49 -> 9.06).
constexpr int kPlaneLoad = 2;

__device__ __forceinline__ void store16(int8_t* row, int k, int K, bool vec, const v4i& v) {
  if (vec && k + 16 <= K) {
    *reinterpret_cast<v4i*>(row + k) = v;
  } else {
    for (int i = 0; i < 16 && k + i < K; ++i) row[k + i] = (int8_t)(v[i >> 2] >> (8 * (i & 3)));
  }
}

// LN (bf16 input only): parameter-free LayerNorm before the quantization. XBUF, int8 input: brick
// and activation loads through buffer resources, straight-line; measured faster for a few tokens
// (4.35 vs 4.58 us at T = 1 on the 2560 -> 6912 decode shape), and with non-temporal brick loads
// at 16 tokens too when the launch is one batch (4.95 vs 5.60 us); the int8 launcher takes it for
// T <= 4 and for one-batch launches. The bf16-input kernel loads its bricks through the buffer
// resource too (4.95 vs 5.06 us per one-kernel step at T = 1). XBUF, bf16 input (T = 1, no
// LayerNorm): the row comes through a buffer resource and the token count is a compile-time 1.
// (Every wave taking the absmax over the whole row itself, with no barrier, was measured slower:
// 6.3 vs 4.8 us, the 4320 waves' requests for the same few KB queue at a few L2 channels.)
//
// OUTL (one token, fp32 output, n_out % 16 == 0, one batch): the row block's k:256 outliers are
// added in the same launch, with the arithmetic of the separate outlier kernel (outliers.hip, 8
// partial sums per row over groups c, c + 8, ..., position order within a group, partials added in
// order c = 0 .. 7, then y = fl32(y0 + fl32(o * step))), so both paths give the same bits. The
// quantized row (bf16 input: the quantized pieces; int8 input: the B operands of token 0, stored
// after the products) and the block's outlier planes are staged in dynamic LDS: [K] x_q bytes, then
// [G k][16] positions, [G k][16] bf16 values, [8][16] partial sums. Each thread issues three
// straight-line loads for the planes with the bricks (G k <= 16 nq <= 64 W pieces of each).
//
// rb: the row block this workgroup computes (of the weight whose planes, scale and output are
// passed); xq_writer: this workgroup writes x_q and a' (FUSED; exactly one workgroup of a launch).
template <int FORM, bool FUSED, bool XVEC, int Q, bool LN, bool XBUF, bool OUTL = false>
__device__ __forceinline__ void gemv_body(
    const uint8_t* __restrict__ mask_plane, const uint8_t* __restrict__ code_plane,
    const Layout& L, const int K, const int nq, const int W, const float* __restrict__ gamma_p,
    const void* __restrict__ xin, int64_t ld_x, int8_t* __restrict__ xq_out, int64_t ld_q,
    float* __restrict__ absmax, int64_t T, void* __restrict__ y, int64_t ld_y, int out_kind,
    float ln_eps, const int64_t rb, const bool xq_writer, const uint8_t* __restrict__ opos = nullptr,
    const uint16_t* __restrict__ oval = nullptr, int KO = 0) {
  static_assert(!OUTL || (XBUF && !LN && (FUSED || XVEC)), "outliers: one-token launches only");
  __shared__ v4i red[kGemvMaxWaves][64];
  __shared__ uint32_t wmax[kGemvMaxWaves][kFusedMaxT / 2];  // token pairs, 16 bits each
  __shared__ double lnsum[FUSED ? kGemvMaxWaves : 1][kFusedMaxT];
  __shared__ double lndev[FUSED ? kGemvMaxWaves : 1][kFusedMaxT];
  __shared__ uint32_t xq_lds[FUSED ? kGemvMaxWaves : 1][kFusedMaxT * 64];
  constexpr bool CMP = compact_form(FORM);
  __shared__ uint32_t clut[CMP ? 256 : 1];  // compact nibble table
  // W: the workgroup's waves (blockDim.x / 64), an argument so that no load of the dispatch's
  // group size delays the first loads; the wave index is uniform; readfirstlane lets it feed the buffer loads' scalar offsets
  // directly (otherwise each load sits in a loop over the lanes' distinct offsets)
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int t = lane & 15, g = lane >> 4;
  const bool tok_ok = t < (int)T;

  uint32_t mask[Q][2], codes[Q][4];
  // With FUSED or XBUF, positional and structured-sparse bricks come through a buffer resource
  // over this row block's quads: a quad past the last reads as zero, so the loads are
  // straight-line code and the compiler's wait counts stay exact (a wait for the activations then
  // does not wait for the bricks behind them). The compact plane always comes this way: a quad
  // takes cq = 512 + 8 csb bytes, and the range ends kCompactSlack bytes past the row block's
  // last quad (the plane has that slack), which covers every lane's three-word sign load.
  const int cq = CMP ? (int)compact_quad_bytes(L.csb) : 1024;
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(code_plane + rb * nq * cq), (short)0,
      CMP ? nq * cq + kCompactSlack : (FORM != kFormKept ? nq * 1024 : 0), kBufDword3);
  auto load_bricks = [&](int qoff) {
#pragma unroll
    for (int i = 0; i < Q; ++i) {
      const int q = qoff + wave + i * W;
      if constexpr (CMP) {
        // the lane's nonzero mask, and the three words holding its csb sign bits
        const v2u mk = __builtin_amdgcn_raw_buffer_load_b64(crs, lane * 8, q * cq, kPlaneLoad);
        const int sbit = lane * L.csb;
        const v3u sg = __builtin_amdgcn_raw_buffer_load_b96(
            crs, kCompactMaskBytes + 4 * (sbit >> 5), q * cq, kPlaneLoad);
        mask[i][0] = mk[0]; mask[i][1] = mk[1];
        codes[i][0] = sg[0]; codes[i][1] = sg[1]; codes[i][2] = sg[2];
        codes[i][3] = (uint32_t)(sbit & 31);
      } else if constexpr (FORM != kFormKept && (FUSED || XBUF)) {
        const v4i c = __builtin_amdgcn_raw_buffer_load_b128(crs, lane * 16, q * 1024, kPlaneLoad);
        codes[i][0] = (uint32_t)c[0]; codes[i][1] = (uint32_t)c[1];
        codes[i][2] = (uint32_t)c[2]; codes[i][3] = (uint32_t)c[3];
        mask[i][0] = mask[i][1] = 0;
      } else if (q < nq) {
        load_brick<FORM>(L, mask_plane, code_plane, ((rb * nq + q) << 6) | lane, mask[i],
                         codes[i]);
      } else {
        mask[i][0] = mask[i][1] = 0;
        codes[i][0] = codes[i][1] = codes[i][2] = codes[i][3] = 0;
      }
    }
  };
  v4i b[Q][4];  // B operands: 16 int8 activations per K slice
  float a_t = 0.0f;     // a' of token t (FUSED, else loaded with the operands)
  // The scales are loaded up front, so the epilogue waits for no memory
  const float gamma = gamma_p[0];
  auto build_lut = [&]() {
    if constexpr (CMP) {
      for (int e = threadIdx.x; e < 256; e += blockDim.x) clut[e] = compact_nibble_entry(e);
    }
  };
  // Outlier planes of this row block (OUTL): piece i of the positions is the 16 rows' bytes of
  // (group, slot) i, pieces of the values are halves (8 rows) of theirs; out-of-range pieces read 0.
  extern __shared__ __attribute__((aligned(16))) uint8_t gemv_dyn[];
  const int G = K >> 8;
  const int npos = OUTL ? G * KO : 0;
  v4i opc[3];
  auto load_outliers = [&]() {
    const int64_t n_out = L.n_out;
    const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(opos + rb * 16), (short)0, (int)(npos * n_out - rb * 16), kBufDword3);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(oval + rb * 16), (short)0, (int)(2 * (npos * n_out - rb * 16)), kBufDword3);
    const int p0 = threadIdx.x, p1 = threadIdx.x + 64 * W;
    opc[0] = __builtin_amdgcn_raw_buffer_load_b128(pr, p0 < npos ? p0 * (int)n_out : (1 << 30), 0, 0);
    opc[1] = __builtin_amdgcn_raw_buffer_load_b128(
        vr, p0 < 2 * npos ? 2 * (p0 >> 1) * (int)n_out + 16 * (p0 & 1) : (1 << 30), 0, 0);
    opc[2] = __builtin_amdgcn_raw_buffer_load_b128(
        vr, p1 < 2 * npos ? 2 * (p1 >> 1) * (int)n_out + 16 * (p1 & 1) : (1 << 30), 0, 0);
  };
  v4i acc = v4i{0, 0, 0, 0};
  // int8 input: the waves take batches of W * Q quads in turn, so any K fits; bf16 input (whose
  // quantization needs the whole row first): one batch
  const int nbatch = FUSED ? 1 : (nq + W * Q - 1) / (W * Q);
  // The first batch is straight-line code (its loads go out first thing); further batches loop.
  auto run_batch = [&](const int qoff, const bool first) {
    if constexpr (!FUSED) {
      load_bricks(qoff);
      if (first) build_lut();
      if constexpr (XVEC && XBUF) {
        // One buffer resource over the T activation rows, straight-line loads: the lanes of a
        // missing token take an offset past the range and read zero, as does the K tail of the last
        // row; a piece past K in another row reads that row's padding or the next row, harmless
        // because the weights there are zero. Offsets stay below 2^31: T <= 16, ld_x <= 2^26.
        const int64_t ext = ((int64_t)T - 1) * ld_x + K;
        const __amdgpu_buffer_rsrc_t xr =
            __builtin_amdgcn_make_buffer_rsrc((void*)xin, (short)0, (int)ext, kBufDword3);
#pragma unroll
        for (int i = 0; i < Q; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int voff = tok_ok ? t * (int)ld_x + 16 * b_chunk<FORM>(g, j) : (1 << 30);
            b[i][j] =
                __builtin_amdgcn_raw_buffer_load_b128(xr, voff, (qoff + wave + i * W) * kQuadK, 0);
          }
        // the outlier planes after the activations, so waiting for these waits for no plane
        if constexpr (OUTL) load_outliers();
      } else {
        const int8_t* xrow = reinterpret_cast<const int8_t*>(xin) + (tok_ok ? t : 0) * ld_x;
#pragma unroll
        for (int i = 0; i < Q; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int k = (qoff + wave + i * W) * kQuadK + 16 * b_chunk<FORM>(g, j);
            b[i][j] = v4i{0, 0, 0, 0};
            if (tok_ok && k < K) b[i][j] = load_x16<XVEC>(xrow, k, K);
          }
      }
      if (first) {
        if (out_kind == SBN_OUT_F32 && tok_ok) a_t = absmax[t];
        if constexpr (CMP) __syncthreads();  // the nibble table
      }
    } else {
      // Lane l quantizes elements 4l .. 4l+3 of every token in each of its quads (one quant4 per
      // token and quad, so no lane idles), then the bytes are regrouped through a wave-local LDS
      // buffer into the B layout (lane (t, g) slice j = bytes 64g + 16j .. +15 of token t).
      const uint16_t* xb = reinterpret_cast<const uint16_t*>(xin);
      // XBUF runs one token; the constant lets the compiler drop the other tokens' code
      const int Tn = XBUF ? 1 : (int)T;  // <= kFusedMaxT; loops below stop at the real token count
      // One resource over the row (XBUF): loads are straight-line, positions past K read zero.
      const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<void*>(xin), (short)0, XBUF ? K * 2 : 0, kBufDword3);
      uint2 xv[Q][kFusedMaxT];
#pragma unroll
      for (int i = 0; i < Q; ++i)
#pragma unroll
        for (int tt = 0; tt < kFusedMaxT; ++tt) {
          const int k = (wave + i * W) * kQuadK + 4 * lane;
          uint2 v = make_uint2(0, 0);
          if constexpr (XBUF) {
            if (tt == 0) {
              const v2u r = __builtin_amdgcn_raw_buffer_load_b64(xr, k < K ? 2 * k : (1 << 30), 0, 0);
              v = make_uint2(r[0], r[1]);
            }
          } else if (tt < Tn && k < K) {
            const uint16_t* row = xb + tt * ld_x;
            if constexpr (XVEC) {
              v = *reinterpret_cast<const uint2*>(row + k);
            } else {
              uint32_t w2[2] = {0, 0};
              for (int u = 0; u < 4 && k + u < K; ++u) w2[u >> 1] |= (uint32_t)row[k + u] << (16 * (u & 1));
              v = make_uint2(w2[0], w2[1]);
            }
          }
          xv[i][tt] = v;
        }
      // The bricks (HBM) go out only once the activations have arrived. Issued behind the weight
      // stream of the whole launch, the activations took longer to come back than the bricks and
      // their quantization sat on the critical path; waiting first, they come back quickly and
      // the quantization below overlaps the brick loads. Same-process A/B on the 2560 -> 6912
      // decode shape, one token: 4.23 -> 3.53 us per step (gate and up grouped: 5.48 -> 5.22 us);
      // with the activations taken as constants (a timing copy) the step took 3.16 us. The
      // scheduling barrier keeps the compiler from moving the brick loads up.
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __builtin_amdgcn_sched_barrier(0);
      load_bricks(0);
      if constexpr (OUTL) load_outliers();
      build_lut();  // published by a barrier below
      if constexpr (LN) {
        // Parameter-free LayerNorm of every token row (as sbn_layernorm_quantize_act): fp64 sum
        // and sum of squared deviations over the wave (DPP), then over the waves (one LDS read per
        // lane and a 16-lane DPP tree, a fixed order); the lane's elements are replaced by their
        // bf16 normalized values.
        double ps[kFusedMaxT], pd[kFusedMaxT];
        float mu32[kFusedMaxT], r32[kFusedMaxT];
#pragma unroll
        for (int tt = 0; tt < kFusedMaxT; ++tt) {
          ps[tt] = 0.0;
          if (tt >= Tn) continue;
#pragma unroll
          for (int i = 0; i < Q; ++i) {
            const uint2 v = xv[i][tt];
            ps[tt] += (double)__uint_as_float(v.x << 16) + (double)__uint_as_float(v.x & 0xFFFF0000u) +
                      (double)__uint_as_float(v.y << 16) + (double)__uint_as_float(v.y & 0xFFFF0000u);
          }
          ps[tt] = wave_sum_f64(ps[tt]);
        }
        if (lane == 0) {
#pragma unroll
          for (int tt = 0; tt < kFusedMaxT; ++tt) lnsum[wave][tt] = ps[tt];
        }
        __syncthreads();
#pragma unroll
        for (int tt = 0; tt < kFusedMaxT; ++tt) {
          pd[tt] = 0.0;
          ps[tt] = 0.0;
          if (tt >= Tn) continue;
          ps[tt] = row16_sum_f64(lane < W ? lnsum[lane][tt] : 0.0);
          ps[tt] /= (double)K;  // the mean
#pragma unroll
          for (int i = 0; i < Q; ++i) {
            const int k = (wave + i * W) * kQuadK + 4 * lane;
            const uint2 v = xv[i][tt];
            const float f[4] = {__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                                __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u)};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              if (k + u < K) {
                const double e = (double)f[u] - ps[tt];
                pd[tt] += e * e;
              }
            }
          }
          pd[tt] = wave_sum_f64(pd[tt]);
        }
        if (lane == 0) {
#pragma unroll
          for (int tt = 0; tt < kFusedMaxT; ++tt) lndev[wave][tt] = pd[tt];
        }
        __syncthreads();
#pragma unroll
        for (int tt = 0; tt < kFusedMaxT; ++tt) {
          mu32[tt] = 0.0f;
          r32[tt] = 0.0f;
          if (tt >= Tn) continue;
          const double d = row16_sum_f64(lane < W ? lndev[lane][tt] : 0.0);
          mu32[tt] = (float)ps[tt];
          r32[tt] = (float)(1.0 / sqrt(d / (double)K + (double)ln_eps));
        }
#pragma unroll
        for (int i = 0; i < Q; ++i) {
          const int k = (wave + i * W) * kQuadK + 4 * lane;
#pragma unroll
          for (int tt = 0; tt < kFusedMaxT; ++tt) {
            if (tt >= Tn || k >= K) continue;
            uint2 z = make_uint2(ln_pair(xv[i][tt].x, mu32[tt], r32[tt]),
                                 ln_pair(xv[i][tt].y, mu32[tt], r32[tt]));
            // positions past K stay zero
            if (k + 4 > K) {
              const int keep = K - k;  // 1 .. 3 valid values
              if (keep < 2) z.x &= 0xFFFFu;
              if (keep < 3) z.y = 0u;
              else z.y &= 0xFFFFu;
            }
            xv[i][tt] = z;
          }
        }
      }
      uint32_t m[kFusedMaxT];
#pragma unroll
      for (int tt = 0; tt < kFusedMaxT; ++tt) {
        m[tt] = 0;
#pragma unroll
        for (int i = 0; i < Q; ++i) m[tt] = max_abs_bf16x2(max_abs_bf16x2(m[tt], xv[i][tt].x),
                                                           xv[i][tt].y);
      }
      // Per-token maxima: two tokens per word (16-bit halves), reduced over the wave (DPP), then
      // over the waves through LDS (one read per lane and a 16-lane DPP tree).
      uint32_t pk[kFusedMaxT / 2];
#pragma unroll
      for (int p2 = 0; p2 < kFusedMaxT / 2; ++p2) {
        pk[p2] = 0;
        if (2 * p2 >= Tn) continue;
        const uint32_t a0 = max(m[2 * p2] & 0xFFFFu, m[2 * p2] >> 16);
        const uint32_t a1 = max(m[2 * p2 + 1] & 0xFFFFu, m[2 * p2 + 1] >> 16);
        pk[p2] = wave_max_u16x2(a0 | (a1 << 16));
      }
      if (lane == 0) {
#pragma unroll
        for (int p2 = 0; p2 < kFusedMaxT / 2; ++p2) wmax[wave][p2] = pk[p2];
      }
      __syncthreads();
      uint32_t am2[kFusedMaxT / 2];
#pragma unroll
      for (int p2 = 0; p2 < kFusedMaxT / 2; ++p2)
        am2[p2] = 2 * p2 < Tn ? row16_max_u16x2(lane < W ? wmax[lane][p2] : 0u) : 0u;
      float s_t[kFusedMaxT];
#pragma unroll
      for (int tt = 0; tt < kFusedMaxT; ++tt) {
        s_t[tt] = 0.0f;
        if (tt >= Tn) continue;
        const uint32_t am = (am2[tt >> 1] >> (16 * (tt & 1))) & 0xFFFFu;
        const float a = fmaxf(__uint_as_float(am << 16), kAbsmaxFloor);
        s_t[tt] = 127.0f / a;
        if (tt == t) a_t = a;
      }
      uint32_t* xs = xq_lds[wave];  // [kFusedMaxT][64] words
      const bool vq = ((uintptr_t)xq_out % 4 == 0) && (ld_q % 4 == 0);
#pragma unroll
      for (int i = 0; i < Q; ++i) {
        const int k = (wave + i * W) * kQuadK + 4 * lane;
#pragma unroll
        for (int tt = 0; tt < kFusedMaxT; ++tt) {
          if (tt >= Tn) continue;
          const uint32_t qw = quant4(xv[i][tt].x, xv[i][tt].y, s_t[tt]);
          xs[tt * 64 + lane] = qw;
          if constexpr (OUTL) {
            if (k < K) reinterpret_cast<uint32_t*>(gemv_dyn)[k >> 2] = qw;  // K % 256 == 0
          }
          if (xq_writer && tt < (int)T && k < K) {
            int8_t* dst = xq_out + tt * ld_q + k;
            if (vq && k + 4 <= K) {
              *reinterpret_cast<uint32_t*>(dst) = qw;
            } else {
              for (int u = 0; u < 4 && k + u < K; ++u) dst[u] = (int8_t)(qw >> (8 * u));
            }
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          b[i][j] = t < kFusedMaxT && tok_ok
                        ? *reinterpret_cast<const v4i*>(xs + (t < kFusedMaxT ? t : 0) * 64 +
                                                        4 * b_chunk<FORM>(g, j))
                        : v4i{0, 0, 0, 0};
      }
      if (xq_writer && wave == 0 && g == 0 && tok_ok) absmax[t] = a_t;
    }

#pragma unroll
    for (int i = 0; i < Q; ++i) {
      if (qoff + wave + i * W < nq) {
        if constexpr (FORM == kFormSparse24) {
#pragma unroll
          for (int blk = 0; blk < 2; ++blk) {
            uint32_t a[4];
            exp_word_to_i8(codes[i][2 * blk], a);
            acc = smfmac16(a, b[i][2 * blk], b[i][2 * blk + 1], codes[i][2 * blk + 1], acc);
          }
        } else {
          uint32_t a[16];
          if constexpr (CMP) {
            const uint32_t sh = codes[i][3];
            const uint32_t lo = __builtin_amdgcn_alignbit(codes[i][1], codes[i][0], sh);
            const uint32_t hi = __builtin_amdgcn_alignbit(codes[i][2], codes[i][1], sh);
            decode_compact<compact_m(FORM)>(mask[i], lo, hi, L.n, L.csb, clut, a);
          } else {
            decode<FORM>(L, mask[i], codes[i], a);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) acc = mfma16(a + 4 * j, b[i][j], acc);
        }
      }
    }
    if constexpr (OUTL && !FUSED) {
      // token 0's activation bytes of this wave's quads into the row copy (one batch: qoff = 0)
      if (t == 0) {
#pragma unroll
        for (int i = 0; i < Q; ++i) {
          const int q = wave + i * W;
          if (q < nq) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              *reinterpret_cast<v4i*>(gemv_dyn + q * kQuadK + 16 * b_chunk<FORM>(g, j)) = b[i][j];
          }
        }
      }
    }
  };
  run_batch(0, true);
  for (int qb = 1; qb < nbatch; ++qb) run_batch(qb * W * Q, false);
  const float step = out_kind == SBN_OUT_F32 ? a_t / 127.0f : 0.0f;
  red[wave][lane] = acc;
  uint8_t* const pos_s = gemv_dyn + K;             // [G k][16]
  uint16_t* const val_s = reinterpret_cast<uint16_t*>(pos_s + 16 * npos);  // [G k][16]
  float* const part_s = reinterpret_cast<float*>(val_s + 16 * npos);       // [8][16]
  if constexpr (OUTL) {
    const int p0 = threadIdx.x, p1 = threadIdx.x + 64 * W;
    if (p0 < npos) *reinterpret_cast<v4i*>(pos_s + 16 * p0) = opc[0];
    if (p0 < 2 * npos) *reinterpret_cast<v4i*>(val_s + 8 * p0) = opc[1];
    if (p1 < 2 * npos) *reinterpret_cast<v4i*>(val_s + 8 * p1) = opc[2];
  }
  __syncthreads();
  if constexpr (OUTL) {
    // unit (c, r): partial sum c of row r of the block
    for (int u = threadIdx.x; u < 128; u += 64 * W) {
      const int r = u & 15, c = u >> 4;
      float o = 0.0f;
      for (int gg = c; gg < G; gg += 8) {
        for (int j = 0; j < KO; ++j) {
          const int gj = gg * KO + j;
          const float v = __uint_as_float((uint32_t)val_s[16 * gj + r] << 16);
          const int8_t xv8 = reinterpret_cast<const int8_t*>(gemv_dyn)[gg * 256 + pos_s[16 * gj + r]];
          o = __fadd_rn(o, __fmul_rn((float)xv8, v));
        }
      }
      part_s[c * 16 + r] = o;
    }
    __syncthreads();
  }
  if (wave != 0 || !tok_ok) return;
  // (A fully unrolled sum over all 16 slots, masked, measured slower than this loop.)
  v4i sum = red[0][lane];
  for (int w = 1; w < W; ++w) sum += red[w][lane];
  const int64_t row0 = rb * 16 + 4 * g;
  if constexpr (OUTL) {
    // y = fl32( fl32(fl32(fl32(acc) * gamma) * step) + fl32(o * step) ), o summed as above
    float* const yr = reinterpret_cast<float*>(y) + row0;
    float f[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float o = part_s[4 * g + i];
#pragma unroll
      for (int cc = 1; cc < 8; ++cc) o = __fadd_rn(o, part_s[cc * 16 + 4 * g + i]);
      f[i] = __fadd_rn(__fmul_rn(__fmul_rn((float)sum[i], gamma), step), __fmul_rn(o, step));
    }
    if (((uintptr_t)yr % 16) == 0) {
      *reinterpret_cast<float4*>(yr) = make_float4(f[0], f[1], f[2], f[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) yr[i] = f[i];
    }
    return;
  }
  const bool vec = ((uintptr_t)y % 16 == 0) && (ld_y % 4 == 0) && row0 + 3 < L.n_out;
  if (vec) {  // the lane's four consecutive rows in one store
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
      if (row < L.n_out) store_out(y, ld_y, out_kind, t, row, sum[i], gamma, step);
    }
  }
}

// Entry of the bf16-input kernels (and of the int8 kernels for other callers): the layout comes by
// value and K and the quad count are read from it.
template <int FORM, bool FUSED, bool XVEC, int Q, bool LN, bool XBUF>
__global__ __launch_bounds__(kGemvMaxWaves * 64) void bitlinear_gemv(
    const uint8_t* __restrict__ mask_plane, const uint8_t* __restrict__ code_plane, Layout L,
    const float* __restrict__ gamma_p, const void* __restrict__ xin, int64_t ld_x,
    int8_t* __restrict__ xq_out, int64_t ld_q, float* __restrict__ absmax, int64_t T,
    void* __restrict__ y, int64_t ld_y, int out_kind, float ln_eps) {
  gemv_body<FORM, FUSED, XVEC, Q, LN, XBUF>(mask_plane, code_plane, L, (int)L.K, (int)L.quads,
                                            (int)(blockDim.x >> 6), gamma_p, xin, ld_x, xq_out,
                                            ld_q, absmax, T, y, ld_y, out_kind, ln_eps,
                                            (int64_t)blockIdx.x, blockIdx.x == 0);
}

// Grouped GEMV: several packed weights that share K, the pattern and the code form, and read the
// same activations (e.g. the Q, K and V projections of a block, or its gate and up projections),
// in one launch. The workgroups of member i are [rb_end[i-1], rb_end[i]); each computes one row
// block of its member with that member's planes, scale and output, exactly as a launch on that
// weight alone would.
constexpr int kMaxGroup = 8;
struct GemvMember {
  const uint8_t* codes;  // code plane (or compact plane) of the member
  const uint8_t* mask;   // mask plane (kept form), or nullptr
  const float* gamma;    // the scale the matmul multiplies by
  void* y;               // output [T][ld_y]
  int64_t ld_y;
  int64_t n_out;
  int rb_end;            // one past the member's last workgroup
};
struct GemvGroup {
  GemvMember m[kMaxGroup];
  int count;
};

// Fills a group from packed weights that share K, the pattern and the code form (not the compact
// plane), each workgroup taking rb_per_wg row blocks of one member; returns the launch's workgroup
// count.
inline int make_group(const sbn_packed* const* hs, int count, void* const* ys,
                      const int64_t* ld_ys, GemvGroup& G, int rb_per_wg = 1) {
  int end = 0;
  for (int i = 0; i < kMaxGroup; ++i) {
    GemvMember& m = G.m[i];
    if (i < count) {
      end += (int)((hs[i]->L.row_blocks + rb_per_wg - 1) / rb_per_wg);
      m = GemvMember{hs[i]->codes, hs[i]->mask, hs[i]->gamma_out(), ys[i], ld_ys[i],
                     hs[i]->L.n_out, end};
    } else {
      m = GemvMember{nullptr, nullptr, nullptr, nullptr, 0, 0, end};
    }
  }
  G.count = count;
  return end;
}

// The member of workgroup b (uniform) and its row block within that member.
__device__ __forceinline__ int group_member(const GemvGroup& G, int b, int64_t& rb) {
  int i = 0;
  while (i + 1 < G.count && b >= G.m[i].rb_end) ++i;
  rb = b - (i > 0 ? G.m[i - 1].rb_end : 0);
  return i;
}

template <int FORM, bool FUSED, bool XVEC, int Q, bool LN, bool XBUF>
__global__ __launch_bounds__(kGemvMaxWaves * 64) void bitlinear_gemv_group(
    GemvGroup G, Layout L, const void* __restrict__ xin, int64_t ld_x,
    int8_t* __restrict__ xq_out, int64_t ld_q, float* __restrict__ absmax, int64_t T,
    int out_kind, float ln_eps) {
  int64_t rb;
  const int i = group_member(G, (int)blockIdx.x, rb);
  Layout Lm = L;
  Lm.n_out = G.m[i].n_out;
  gemv_body<FORM, FUSED, XVEC, Q, LN, XBUF>(G.m[i].mask, G.m[i].codes, Lm, (int)L.K,
                                            (int)L.quads, (int)(blockDim.x >> 6), G.m[i].gamma,
                                            xin, ld_x, xq_out, ld_q, absmax, T, G.m[i].y,
                                            G.m[i].ld_y, out_kind, ln_eps, rb, blockIdx.x == 0);
}

// The one-token bf16 step with the k:256 outlier term (fp32 output; planes [G k][n_out]).
template <int FORM, int Q>
__global__ __launch_bounds__(kGemvMaxWaves * 64) void bitlinear_gemv_outl(
    const uint8_t* __restrict__ mask_plane, const uint8_t* __restrict__ code_plane, Layout L,
    const float* __restrict__ gamma_p, const void* __restrict__ xin, int8_t* __restrict__ xq_out,
    int64_t ld_q, float* __restrict__ absmax, void* __restrict__ y,
    const uint8_t* __restrict__ opos, const uint16_t* __restrict__ oval, int KO) {
  gemv_body<FORM, true, true, Q, false, true, true>(
      mask_plane, code_plane, L, (int)L.K, (int)L.quads, (int)(blockDim.x >> 6), gamma_p, xin,
      (int64_t)L.K, xq_out, ld_q, absmax, 1, y, (int64_t)L.n_out, SBN_OUT_F32, 0.0f,
      (int64_t)blockIdx.x, blockIdx.x == 0, opos, oval, KO);
}

// Dynamic LDS of bitlinear_gemv_outl.
inline size_t gemv_outl_smem(int64_t K, int KO) {
  return (size_t)K + (size_t)(K >> 8) * (size_t)KO * 48 + 8 * 16 * sizeof(float);
}

}  // namespace
}  // namespace sbn
