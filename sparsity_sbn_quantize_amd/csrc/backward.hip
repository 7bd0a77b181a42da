// Data gradient of the BitLinear layer under the straight-through estimator.
//
// "Microsoft BitNet 1.58: The Era of 1-Bit Large Language Models", section "Training with the
// Straight-Through Estimator": the backward pass treats the quantizers as the identity, while
// the forward uses the ternary weights of section "The BitLinear Layer" (gamma times the codes).
// With y = x (gamma C)^T the data gradient is therefore
//
//   dX[t][k] = fl32( gamma * sum_r dY[t][r] * C[r][k] )
//
// with C the handle's ternary codes (0 at pruned positions). dY is bf16; every product with a
// code in {-1, 0, +1} is exact and the sums are fp32 (bf16 MFMA, fp32 accumulation).
//
// The reduction runs over the weight rows, so the A operand needs, per lane, 8 consecutive rows
// of one column: the transposed code plane (pack.hip) stores exactly that, 2 bits per weight.
// A workgroup of W = 4 waves computes 256 columns x 128 tokens (W = 8: 512 columns, for launches
// with many tiles, so that each dY tile below serves twice the MFMAs); wave w owns 4 column
// fragments (64 columns) and all 128 tokens. Each step covers 128 rows: the 128 x 128 bf16 dY tile goes global -> LDS
// directly into a 2-slot ring one step ahead (the same [token group][16-byte chunk][token] layout
// as the forward's activations, free of bank conflicts), the transposed bricks come one step
// ahead into registers, and slice j+1 (32 rows) is decoded to bf16 while the MFMAs of slice j run.
#include "sbn_internal.hpp"

namespace sbn {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBwCF = 4;                                 // 16-column fragments per wave
constexpr int kBwTF = 8;                                 // 16-token fragments per tile
constexpr int kBwTok = kBwTF * 16;                       // 128 tokens per tile
constexpr int kBwStepRows = 128;                         // rows per step (4 MFMA slices of 32)
constexpr int kBwTileBytes = kBwTok * kBwStepRows * 2;   // dY tile of one step (32 KB)
constexpr int kBwWideMinTiles = 200;  // 8-wave tiles (512 columns) when there are this many
constexpr size_t kBwSmem = 2 * (size_t)kBwTileBytes;
// Lane offset that lies past every buffer range the dY loads use: such pieces read as zero.
constexpr int kDxPolicy = 1 | 2 | 16;  // buffer cache-policy bits sc0 | nt | sc1: dX stores
constexpr int kOutOfRange = 0x7FFFFFF0;
// Largest dY extent (bytes from a tile's first row to the end of the data) of the buffer path.
constexpr int64_t kMaxBufExtent = 0x7FFF0000;

// bf16 A operand of MFMA slice s (0, 1) of transposed word w: dword p holds rows 2p and 2p + 1 of
// the slice. The 2-bit codes (0, 1 = +1, 2 = -1) become selectors: x = (c0 | c1 << 16),
// x * 0x101 + 0x40004 = bytes [c0 + 4, c0, c1 + 4, c1], which v_perm maps to the low bytes
// {0x00, 0x80, 0x80} and high bytes {0x00, 0x3F, 0xBF} of bf16 {0, +1, -1}.
__device__ __forceinline__ uint32_t tdecode1(uint32_t w, int s, int p) {
  const uint32_t x = (w >> (8 * s + 2 * p)) & 0x00030003u;
  return __builtin_amdgcn_perm(0x00808000u, 0x00BF3F00u, x * 0x0101u + 0x00040004u);
}
__device__ __forceinline__ void tdecode(uint32_t w, int s, uint32_t out[4]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) out[p] = tdecode1(w, s, p);
}

__device__ __forceinline__ v4f mfma_bf16(const uint32_t a[4], v4i b, v4f c) {
  const v4i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av),
                                                 __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

template <bool XVEC, int W>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bitlinear_bwd_dx(const uint32_t* __restrict__ tplane, int rq_count, int64_t n_out, int64_t K,
                      const float* __restrict__ gamma_p, const uint16_t* __restrict__ dy,
                      int64_t ld_dy, int64_t T, float* __restrict__ dx, int64_t ld_dx,
                      int tiles_c, int tiles_t, uint32_t* __restrict__ pack_gen) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // The transposed plane this launch reads was built from the handle's last pack (the transpose
  // kernel ran just before, in stream order); record that pack count for the next call.
  if (blockIdx.x == 0 && threadIdx.x == 0) pack_gen[1] = pack_gen[0];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int lin = xcd_order((int)gridDim.x, (int)blockIdx.x);
  int tile_c, tile_t;
  grouped_tile(lin, tiles_c, tiles_t, tile_c, tile_t);
  constexpr int kBwXLoads = kBwTileBytes / 16 / (W * 64);  // 16-byte pieces per thread per step
  const int64_t cb0 = (int64_t)tile_c * (W * kBwCF) + wave * kBwCF;  // first column fragment
  const int64_t t0 = (int64_t)tile_t * kBwTok;

  // Transposed bricks: slot (cb * rq_count + rq) * 64 + lane, 8 bytes; the wave's 4 column
  // fragments are rq_count * 512 bytes apart.
  // The plane holds the column fragments of whole 256-column quads; with 512-column tiles the
  // waves of a last tile's second half may lie wholly past it: their resource is empty (every
  // brick reads zero) and their columns are never stored.
  const int64_t plane_cf = (K + 255) / 256 * 16;
  const __amdgpu_buffer_rsrc_t trs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(tplane + cb0 * rq_count * 128), (short)0, cb0 < plane_cf ? 0x7FFFFFFF : 0,
      kBufDword3);
  const int cf_bytes = rq_count * 512;
  typedef uint32_t TBricks[kBwCF][2];
  auto load_t = [&](int rq, TBricks& tw) {
#pragma unroll
    for (int cf = 0; cf < kBwCF; ++cf) {
      const v2u v = __builtin_amdgcn_raw_buffer_load_b64(trs, lane * 8, cf * cf_bytes + rq * 512, 0);
      tw[cf][0] = v[0];
      tw[cf][1] = v[1];
    }
  };

  // dY pieces: wave-instruction ii covers token group ii / 4 and 16-byte chunks 4 (ii % 4) ..
  // +3; lane l takes token l % 16 and chunk 4 (ii % 4) + l / 16 (rows 8 chunk .. +7 of the step)
  // and lands at 1 KB-block ii + 16 l of the slot. The buffer path reads through resources whose
  // range ends with the last token's row; pieces of rows past n_out get an out-of-range lane
  // offset, and both read as zero (n_out is a multiple of 8 there). The other path gathers the
  // 8 values with bounds checks. Tokens past T are never stored.
  const uint8_t* const y0 = reinterpret_cast<const uint8_t*>(dy) + t0 * ld_dy * 2;
  const int64_t row_bytes = ld_dy * 2;
  const int64_t y_extent = (T - 1 - t0) * row_bytes + n_out * 2;
  const int ylane = (lane & 15) * (int)row_bytes + (lane >> 4) * 16;
  auto load_dy = [&](int rq, int slot) {
    uint8_t* dst = smem + slot * kBwTileBytes + wave * (kBwXLoads * 1024);
    // One buffer resource per step (based at the step's first row of the tile's first token);
    // the piece's place in the tile is a lane offset, below T ld_dy 2 < kMaxBufExtent.
    const int64_t left = y_extent - (int64_t)rq * 256;
    const int nrec = left <= 0 ? 0 : (int)left;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(y0 + (int64_t)rq * 256), (short)0, nrec, kBufDword3);
    const int rowb = (int)row_bytes;
#pragma unroll
    for (int i = 0; i < kBwXLoads; ++i) {
      const int ii = wave * kBwXLoads + i, tg = ii >> 2, c0 = (ii & 3) * 4;
      const int64_t r_first = (int64_t)rq * kBwStepRows + 8 * (c0 + (lane >> 4));
      if constexpr (XVEC) {
        const int voff = r_first < n_out ? ylane + tg * 16 * rowb + c0 * 16 : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)(dst + i * 1024), 16, voff, 0, 0,
                                                 0);
      } else {
        const int64_t t = t0 + tg * 16 + (lane & 15);
        uint32_t v[4] = {0u, 0u, 0u, 0u};
        if (t < T) {
          const uint16_t* row = dy + t * ld_dy;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (r_first + e < n_out) v[e >> 1] |= (uint32_t)row[r_first + e] << (16 * (e & 1));
        }
        const v4i pv = {(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
        *reinterpret_cast<v4i*>(dst + i * 1024 + lane * 16) = pv;
      }
    }
  };

  v4f acc[kBwCF][kBwTF];
#pragma unroll
  for (int cf = 0; cf < kBwCF; ++cf)
#pragma unroll
    for (int tf = 0; tf < kBwTF; ++tf) acc[cf][tf] = v4f{0.f, 0.f, 0.f, 0.f};
  // fragment read offset of lane (t, g): chunk 4g + j (rows 32g + 8j ..) of token t
  const int rlane = (lane >> 4) * 1024 + (lane & 15) * 16;
  typedef uint32_t ASlice[kBwCF][4];
  auto decode_slice = [&](const TBricks& tw, int j, ASlice& out) {
#pragma unroll
    for (int cf = 0; cf < kBwCF; ++cf) tdecode(tw[cf][j >> 1], j & 1, out[cf]);
  };

  if (rq_count > 0) {
    TBricks b0, b1;
    ASlice a0, a1;
    load_t(0, b0);
    load_dy(0, 0);
    load_t(rq_count > 1 ? 1 : 0, b1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // ring slot of step 0 written
    __syncthreads();
    decode_slice(b0, 0, a0);
    // Step rq: the dY tile of step rq+1 goes out first (past the last step every piece reads
    // zero and the slot is never read); MFMA group j (slice j: 4 column x 8 token fragments)
    // runs while slice j+1 is decoded (slice 0 of step rq+1 during group 3); then the bricks of
    // step rq+2 are loaded. Before the closing barrier each wave waits for its dY pieces; only
    // the brick loads issued after them may still be in flight.
    auto step = [&](int rq, int slot, TBricks& bcur, const TBricks& bnext) {
      load_dy(rq + 1, slot ^ 1);
      __builtin_amdgcn_sched_barrier(0);
      const uint8_t* xt = smem + slot * kBwTileBytes + rlane;
      v4i bv = *reinterpret_cast<const v4i*>(xt);
      // Fenced groups (as the forward GEMM): group (j, tf) issues the LDS read of the next
      // group's dY first, then its 4 MFMAs, then its two of the next slice's 16 decoded words, and
      // nothing crosses the fence after it, so every read is one group ahead of its MFMAs.
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ASlice& cur = (j & 1) ? a1 : a0;
        ASlice& nxt = (j & 1) ? a0 : a1;
        const TBricks& src = j < 3 ? bcur : bnext;
        const int sj = j < 3 ? j + 1 : 0;
#pragma unroll
        for (int tf = 0; tf < kBwTF; ++tf) {
          const int nj = tf + 1 < kBwTF ? j : j + 1, ntf = tf + 1 < kBwTF ? tf + 1 : 0;
          v4i bn = bv;
          if (nj < 4) bn = *reinterpret_cast<const v4i*>(xt + ntf * 4096 + nj * 256);
#pragma unroll
          for (int cf = 0; cf < kBwCF; ++cf) acc[cf][tf] = mfma_bf16(cur[cf], bv, acc[cf][tf]);
#pragma unroll
          for (int e = tf * 4 * kBwCF / kBwTF; e < (tf + 1) * 4 * kBwCF / kBwTF; ++e)
            nxt[e >> 2][e & 3] = tdecode1(src[e >> 2][sj >> 1], sj & 1, e & 3);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // LDS read
          __builtin_amdgcn_sched_group_barrier(0x008, kBwCF, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);     // VALU
          __builtin_amdgcn_sched_barrier(0);
          bv = bn;
        }
      }
      load_t(rq + 2 < rq_count ? rq + 2 : rq_count - 1, bcur);
      if (XVEC) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kBwCF));
      } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      }
      __syncthreads();
    };
    int rq = 0;
    for (; rq + 1 < rq_count; rq += 2) {
      step(rq, 0, b0, b1);
      step(rq + 1, 1, b1, b0);
    }
    if (rq < rq_count) step(rq, 0, b0, b1);
  }

  // Each lane holds 4 consecutive columns of one token per (cf, tf).
  const float gamma = gamma_p[0];
  const bool vec_out = (((uintptr_t)dx | (uintptr_t)(ld_dx * 4)) & 15) == 0;
  // Vector stores: a buffer resource based at the tile's first token row (32-bit offsets while
  // ld_dx < 2^22, plain global stores beyond), written through (sc0 nt sc1). Same-process A/B
  // against plain global stores on the 7B FFN shapes at T = 8192: 562 -> 549 us (up), 580 -> 577
  // us (down).
  const bool dbuf = ld_dx < (int64_t{1} << 22);
  const __amdgpu_buffer_rsrc_t dro =
      __builtin_amdgcn_make_buffer_rsrc(dx + t0 * ld_dx, (short)0, 0x7FFFFFFF, kBufDword3);
#pragma unroll
  for (int tf = 0; tf < kBwTF; ++tf) {
    const int64_t t = t0 + tf * 16 + (lane & 15);
    if (t >= T) continue;
#pragma unroll
    for (int cf = 0; cf < kBwCF; ++cf) {
      const int64_t k0 = (cb0 + cf) * 16 + 4 * (lane >> 4);
      const v4f v = acc[cf][tf];
      float* const o = dx + t * ld_dx + k0;
      if (vec_out && k0 + 4 <= K) {
        v4i f;
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = (int)__float_as_uint(__fmul_rn(v[i], gamma));
        if (dbuf) {
          __builtin_amdgcn_raw_buffer_store_b128(f, dro, (int)(((t - t0) * ld_dx + k0) * 4), 0,
                                                 kDxPolicy);
        } else {
          *reinterpret_cast<v4i*>(o) = f;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (k0 + i < K) o[i] = __fmul_rn(v[i], gamma);
      }
    }
  }
}

}  // namespace

hipError_t launch_bwd_dx(const sbn_packed* h, const uint16_t* dy, int64_t ld_dy, int64_t T,
                         float* dx, int64_t ld_dx, hipStream_t s) {
  const Layout& L = h->L;
  // The transposed plane is rebuilt when a pack has run since it was last built; the check is
  // made on the device (pack counts in the handle), so it holds when packs or data gradients are
  // replayed from captured graphs. An up-to-date plane costs one launch whose workgroups exit.
  if (h->rq_count > 0) {
    hipError_t e = launch_transpose_codes(h, s);
    if (e != hipSuccess) return e;
  }
  const int64_t tiles_t = (T + kBwTok - 1) / kBwTok;
  const bool xvec = ((uintptr_t)dy % 16 == 0) && (ld_dy % 8 == 0) && (L.n_out % 8 == 0) &&
                    (double)T * (double)ld_dy * 2.0 < (double)kMaxBufExtent;
  // 512 columns per tile (8 waves) when such tiles number kBwWideMinTiles: each step's dY tile
  // then goes to LDS once for 512 columns instead of once per 256 (as the forward GEMM)
  const int64_t tiles_c8 = (L.quads + 1) / 2;
  const bool w8 = xvec && tiles_c8 * tiles_t >= kBwWideMinTiles;
  const int64_t tiles_c = w8 ? tiles_c8 : L.quads;
#define SBN_BWD(XV, WW)                                                                        \
  do {                                                                                         \
    hipError_t e = allow_smem(bitlinear_bwd_dx<XV, WW>, kBwSmem);                              \
    if (e != hipSuccess) return e;                                                             \
    hipLaunchKernelGGL((bitlinear_bwd_dx<XV, WW>), dim3((unsigned)(tiles_c * tiles_t)),          \
                       dim3(WW * 64), kBwSmem, s, h->tplane, (int)h->rq_count, L.n_out, L.K,     \
                       h->gamma_out(), dy, ld_dy, T, dx, ld_dx, (int)tiles_c, (int)tiles_t,     \
                       h->pack_gen);                                                           \
  } while (0)
  if (w8) {
    SBN_BWD(true, 8);
  } else if (xvec) {
    SBN_BWD(true, 4);
  } else {
    SBN_BWD(false, 4);
  }
#undef SBN_BWD
  return hipGetLastError();
}

}  // namespace sbn
