// Host-side internals of libsbn: the packed-weight handle and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "sbn.h"
#include "sbn_common.hpp"

struct sbn_packed {
  sbn::Layout L;
  size_t code_row_bytes, mask_row_bytes;  // reference packed format (RPF) row sizes
  size_t mask_plane_bytes, code_plane_bytes;
  int num_partials;    // absmean partial sums (one per block of the reduction kernel)
  uint8_t* base;       // single device allocation holding everything below
  size_t base_bytes;
  uint8_t* mask;       // mask plane (brick fragments), or nullptr when n == m
  uint8_t* codes;      // code plane (brick fragments)
  float* gamma;        // device scalar
  double* partials;    // device workspace [num_partials]
  uint32_t* gemm_sync;  // split-K words: kGemmSyncInts (two per slot, never reset), then the
                        // give-up counter
  uint32_t* kx_count;   // large-K GEMV split over K: one arrival counter per 256-row group (in
                        // the split-K words' region, reset by each group's last arrival)
  uint8_t* kx_part;     // its int32 partial sums, 16 KB per (row group, K chunk)
  int kx_chunks;        // K chunks of that split (0: the layout has none)
  int splitk_spin_limit;  // s_sleep rounds before a waiting split-K half gives up
  int splitk_publish;     // 1; 0 only in the test mode that withholds the partial sums
  uint32_t* flip_parts;  // keep bits changed by the last pack, one count per pack wave
  uint32_t* vc_parts;   // variance correction: nonzero counts (dense, n:m) per pack wave
  float* gamma_vc;      // variance-corrected output scale (device scalar)
  bool vc;              // the last pack applied the variance correction (host-side state)
  uint32_t* tplane;     // transposed code plane (data-gradient matmul), 2 bits per weight
  int64_t rq_count;     // 128-row groups of the transposed plane
  uint32_t* pack_gen;   // device words: [0] packs of this handle, [1] the pack count the
                        // transposed plane was built from (graph replays of a pack keep it right)
  uint8_t* cplane;      // compact plane (nonzero masks + sign slots), read by the GEMV
  size_t cplane_bytes;  // its size, the slack included
  size_t compact_row_bytes;  // per-row bytes of the compact export stream
  bool compact;         // the last pack wrote the compact plane (host-side state)
  int outlier_k;        // k of the last pack's k:256 outliers (0: none; host-side state)
  bool outlier_planes;  // the planes below exist (K % 256 == 0)
  uint8_t* opos;        // outlier positions [K/256][16][n_out] (k of the 16 slots used)
  uint16_t* oval;       // outlier bf16 values, same layout
  unsigned long long* omask;  // outlier positions as one 64-bit word per brick slot
  double* osum;         // outlier |w| sums, one per selection workgroup of 256 groups
  double* band_part;     // single-pass re-pack: gamma's partial sum per fragment
  uint8_t* band_seg;     // per fragment: the count of listed pieces (kept magnitudes near the
                         // old threshold), then the pieces (kBandRecBytes per fragment)
  uint32_t* band_lim;    // the bracket [T_lo, T_hi] the pass used (fp32 bit patterns), the
                         // fixed-point overflow flag, the fix-up kernel's arrival counter
  unsigned long long* band_slots;  // gamma's fixed-point sum, kBandSlots counters 128 B apart
  bool gamma_valid;      // gamma holds a previous pack's value (host-side state)
  bool single_pass;      // the last pack read the latent weights once (host-side state)
  int device;
  bool async_alloc;     // base came from hipMallocAsync (released with hipFreeAsync)
  hipStream_t last_stream;
  // Scale the matmuls multiply by: gamma, or the variance-corrected gamma.
  float* gamma_out() const { return vc ? gamma_vc : gamma; }
};

namespace sbn {

// Sets the calling thread's sbn_last_error() message (printf format) and returns `code`.
sbn_status set_error(sbn_status code, const char* fmt, ...);

// Words of split-K handshake a handle holds (2 per wave of up to 256 tiles x 4 waves); the
// give-up counter follows them.
constexpr int kGemmSyncInts = 256 * 4 * 2;
// Large-K GEMV split over K (5 to 16 tokens, 49 to 128 quads): quads per K chunk, and the row
// groups (16 row blocks each) rounded up to a multiple of the 8 XCDs.
constexpr int kKxQuads = 7;
constexpr int kKxMinQuads = 49, kKxMaxQuads = 128;
inline int64_t kx_row_groups(int64_t row_blocks) { return ((row_blocks + 15) / 16 + 7) / 8 * 8; }
// s_sleep rounds a waiting split-K half spins before it gives up (its partner is already past its
// main loop, so this is never reached in a correct run).
constexpr int kSplitSpinLimit = 1 << 24;
// Single-pass re-pack: bytes of a fragment's record (the listed-piece count, then the pieces)
// and the pieces it can list for the fix-up kernel.
constexpr int kBandRecBytes = 128;
constexpr int kBandSegCap = kBandRecBytes - 4;
// Counters of the single pass's fixed-point absmean sum (fragment f adds to counter f % 64).
constexpr int kBandSlots = 64;

// The device memory layout of a handle for an (n_out, K, n:m) weight: offsets of the planes and
// words in one allocation. The regions below forward_bytes are all that the pack (without the
// compact or outlier options) and the forward use.
struct Plan {
  Layout L;
  int num_partials;
  int64_t rq_count;
  bool oplanes;
  size_t mask_bytes, code_bytes, cplane_bytes;
  size_t off_mask, off_codes, off_gamma, off_part, off_sync, off_flips, off_vc, off_gamma_vc,
      off_tplane, off_cplane, off_opos, off_oval, off_omask, off_osum, off_kx, off_band;
  int kx_chunks;
  int gen_index;  // the pack-generation words, in the split-K words' region
  size_t forward_bytes, total_bytes;
};
size_t align_up(size_t v, size_t a);
sbn_status make_plan(int64_t n_out, int64_t K, int n, int m, Plan& p);
// Points the handle's planes into `base` (laid out by the plan) and sets its defaults.
void bind_planes(sbn_packed& h, const Plan& p, uint8_t* base);
// The split-K test settings from the environment (SBN_SPLITK_SPIN_LIMIT, SBN_SPLITK_WITHHOLD).
void splitk_settings(int& spin_limit, int& publish);

// Number of blocks of the absmean reduction for a tensor with n_out rows (fixed per shape, so the
// fp64 partial-sum order, and hence gamma, is reproducible run to run).
int absmean_blocks(int64_t n_out);

hipError_t launch_quantize_act(const uint16_t* x, int64_t T, int64_t K, int64_t ld_x, int8_t* q,
                               int64_t ld_q, float* absmax, hipStream_t s);
hipError_t launch_ln_quantize_act(const uint16_t* x, int64_t T, int64_t K, int64_t ld_x,
                                  float eps, int8_t* q, int64_t ld_q, float* absmax,
                                  hipStream_t s);
hipError_t launch_pack(const float* w, int64_t ld_w, sbn_packed* h, hipStream_t s);
hipError_t launch_export(const sbn_packed* h, int8_t* codes, uint8_t* keep, float* gamma,
                         hipStream_t s);
hipError_t launch_export_rpf(const sbn_packed* h, uint8_t* code_bytes, uint8_t* mask_bytes,
                             hipStream_t s);
hipError_t launch_bitlinear(const sbn_packed* h, const int8_t* xq, int64_t ld_q,
                            const float* absmax, int64_t T, void* y, int64_t ld_y, int out_kind,
                            hipStream_t s);
hipError_t launch_export_compact(const sbn_packed* h, uint8_t* out, hipStream_t s);
int rank_bits(int n, int m);  // ceil(log2 C(m, n))
// One-token int8 GEMV with the k:256 outlier term in the same launch (gemv_i8.hip), and whether a
// call fits it (outliers, T = 1, fp32 output checked by the caller, n_out % 16 == 0, one batch).
bool gemv_int8_outl_fits(const sbn_packed* h, const int8_t* xq, int64_t T);
hipError_t launch_gemv_int8_outl(const sbn_packed* h, const int8_t* xq, const float* absmax,
                                 float* y, hipStream_t s);
hipError_t launch_export_rank(const sbn_packed* h, uint8_t* out, hipStream_t s);
hipError_t launch_outlier_select(const float* w, int64_t ld_w, const sbn_packed* h, hipStream_t s);
hipError_t launch_outlier_add(const sbn_packed* h, const int8_t* xq, int64_t ld_q,
                              const float* absmax, int64_t T, float* y, int64_t ld_y,
                              hipStream_t s);
hipError_t launch_export_outliers(const sbn_packed* h, uint8_t* pos, uint16_t* val,
                                  hipStream_t s);
// The int8-input GEMV (T <= 16, any K), every code form.
hipError_t launch_gemv_int8(const sbn_packed* h, const int8_t* xq, int64_t ld_q,
                            const float* absmax, int64_t T, void* y, int64_t ld_y, int out_kind,
                            hipStream_t s);
hipError_t launch_sum_flips(const sbn_packed* h, uint64_t* out, hipStream_t s);
hipError_t launch_transpose_codes(const sbn_packed* h, hipStream_t s);
hipError_t launch_bwd_dx(const sbn_packed* h, const uint16_t* dy, int64_t ld_dy, int64_t T,
                         float* dx, int64_t ld_dx, hipStream_t s);
// The one-token quantize-and-multiply step without a LayerNorm (gemv_bf16.hip), and whether a
// call fits it (T = 1, no compact plane, x 8-byte aligned, K % 4 == 0, one batch of quads).
bool gemv_bf16_one_fits(const sbn_packed* h, const uint16_t* x, int64_t T, float ln_eps);
hipError_t launch_gemv_bf16_one(const sbn_packed* h, const uint16_t* x, int8_t* xq, int64_t ld_q,
                                float* absmax, void* y, int64_t ld_y, int out_kind,
                                hipStream_t s);
// ln_eps > 0: parameter-free LayerNorm (with that epsilon) before the quantization.
hipError_t launch_bitlinear_bf16(const sbn_packed* h, const uint16_t* x, int64_t ld_x, int64_t T,
                                 int8_t* xq, int64_t ld_q, float* absmax, void* y, int64_t ld_y,
                                 int out_kind, float ln_eps, hipStream_t s);

// Grouped launches over weights that share K, the pattern and the code form (no compact plane,
// no outlier term; checked by the caller): the int8 GEMV (T <= 16) and the one-kernel bf16 step
// (gemv_group_fused_fits). ys, ld_ys: host arrays of the members' outputs.
hipError_t launch_gemv_int8_group(const sbn_packed* const* hs, int count, const int8_t* xq,
                                  int64_t ld_q, const float* absmax, int64_t T, void* const* ys,
                                  const int64_t* ld_ys, int out_kind, hipStream_t s);
bool gemv_group_fused_fits(const sbn_packed* h0, const uint16_t* x, int64_t ld_x, int64_t T);
hipError_t launch_gemv_group_bf16(const sbn_packed* const* hs, int count, const uint16_t* x,
                                  int64_t ld_x, int64_t T, int8_t* xq, int64_t ld_q,
                                  float* absmax, void* const* ys, const int64_t* ld_ys,
                                  int out_kind, float ln_eps, hipStream_t s);

// Raises a kernel's dynamic-LDS limit once per process and kernel (gfx950 has 160 KB of LDS per
// CU).
// A fixed table (no heap allocation: the launchers also serve the entry point that allocates
// nothing); a kernel past the table's end just sets its attribute on every launch.
inline hipError_t allow_smem_ptr(const void* kernel, size_t bytes) {
  static std::mutex mu;
  constexpr int kSlots = 256;
  static const void* done_k[kSlots];
  static size_t done_b[kSlots];
  static int count = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < count; ++i)
    if (done_k[i] == kernel && done_b[i] >= bytes) return hipSuccess;
  hipError_t e =
      hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess && count < kSlots) {
    done_k[count] = kernel;
    done_b[count] = bytes;
    ++count;
  }
  return e;
}
template <typename K>
hipError_t allow_smem(K kernel, size_t bytes) {
  return allow_smem_ptr(reinterpret_cast<const void*>(kernel), bytes);
}

}  // namespace sbn
