// Host-side internals of libsbn: the packed-weight handle and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <utility>
#include <vector>

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
  int* gemm_sync;      // split-K flags: kGemmSyncInts words, zero between calls
  uint32_t* flip_parts;  // keep bits changed by the last pack, one count per pack wave
  uint32_t* vc_parts;   // variance correction: nonzero counts (dense, n:m) per pack wave
  float* gamma_vc;      // variance-corrected output scale (device scalar)
  bool vc;              // the last pack applied the variance correction (host-side state)
  uint32_t* tplane;     // transposed code plane (data-gradient matmul), 2 bits per weight
  int64_t rq_count;     // 128-row groups of the transposed plane
  bool tplane_valid;    // the transposed plane matches the last pack (host-side state)
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
  int device;
  hipStream_t last_stream;
  // Scale the matmuls multiply by: gamma, or the variance-corrected gamma.
  float* gamma_out() const { return vc ? gamma_vc : gamma; }
};

namespace sbn {

// Words of split-K handshake flags a handle holds (2 per wave of up to 256 tiles x 4 waves).
constexpr int kGemmSyncInts = 256 * 4 * 2;

// Number of blocks of the absmean reduction for a tensor with n_out rows (fixed per shape, so the
// fp64 partial-sum order, and hence gamma, is reproducible run to run).
int absmean_blocks(int64_t n_out);

hipError_t launch_quantize_act(const uint16_t* x, int64_t T, int64_t K, int64_t ld_x, int8_t* q,
                               int64_t ld_q, float* absmax, hipStream_t s);
hipError_t launch_ln_quantize_act(const uint16_t* x, int64_t T, int64_t K, int64_t ld_x,
                                  float eps, int8_t* q, int64_t ld_q, float* absmax,
                                  hipStream_t s);
hipError_t launch_pack(const float* w, int64_t ld_w, const sbn_packed* h, hipStream_t s);
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
// ln_eps > 0: parameter-free LayerNorm (with that epsilon) before the quantization.
hipError_t launch_bitlinear_bf16(const sbn_packed* h, const uint16_t* x, int64_t ld_x, int64_t T,
                                 int8_t* xq, int64_t ld_q, float* absmax, void* y, int64_t ld_y,
                                 int out_kind, float ln_eps, hipStream_t s);

// Raises a kernel's dynamic-LDS limit once per process and kernel (gfx950 has 160 KB of LDS per
// CU).
inline hipError_t allow_smem_ptr(const void* kernel, size_t bytes) {
  static std::mutex mu;
  static std::vector<std::pair<const void*, size_t>> done;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& d : done)
    if (d.first == kernel && d.second >= bytes) return hipSuccess;
  hipError_t e =
      hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done.emplace_back(kernel, bytes);
  return e;
}
template <typename K>
hipError_t allow_smem(K kernel, size_t bytes) {
  return allow_smem_ptr(reinterpret_cast<const void*>(kernel), bytes);
}

}  // namespace sbn
