// C ABI of libsbn: argument validation, handle lifecycle and dispatch. Every argument check
// happens before the first HIP call, so a rejected call leaves the GPU untouched.
#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <new>

#include "sbn_internal.hpp"

namespace {

thread_local char g_last_error[512] = "";

sbn_status fail(sbn_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

}  // namespace

namespace sbn {
sbn_status set_error(sbn_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}
}  // namespace sbn

namespace {

sbn_status hip_fail(hipError_t e, const char* what) {
  return fail(SBN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool pattern_ok(int n, int m) { return (m == 4 || m == 8 || m == 16) && n >= 1 && n <= m; }

// The matmul kernels form 32-bit offsets of up to 16 activation rows.
constexpr int64_t kMaxLdQ = (int64_t)1 << 26;

// Shared body of the bf16-input forwards (ln_eps > 0: LayerNorm before the quantization).
sbn_status fwd_bf16(const char* name, const sbn_packed* w, const uint16_t* x_bf16, int64_t ld_x,
                    int64_t T, float ln_eps, int8_t* x_q, int64_t ld_q, float* x_absmax, void* y,
                    int64_t ld_y, sbn_out_kind out_kind, void* stream) {
  if (!w) return fail(SBN_ERR_INVALID_ARG, "%s: handle is null", name);
  if (out_kind != SBN_OUT_F32 && out_kind != SBN_OUT_I32_ACC)
    return fail(SBN_ERR_INVALID_ARG, "%s: out_kind=%d", name, (int)out_kind);
  if (T < 0) return fail(SBN_ERR_INVALID_ARG, "%s: T=%lld < 0", name, (long long)T);
  if (T > INT32_MAX) return fail(SBN_ERR_UNSUPPORTED, "%s: T too large", name);
  if (ld_x < w->L.K || ld_q < w->L.K)
    return fail(SBN_ERR_INVALID_ARG, "%s: ld_x=%lld / ld_q=%lld < K=%lld", name,
                (long long)ld_x, (long long)ld_q, (long long)w->L.K);
  if (ld_q > kMaxLdQ)
    return fail(SBN_ERR_UNSUPPORTED, "%s: ld_q=%lld > %lld", name, (long long)ld_q,
                (long long)kMaxLdQ);
  if (ld_y < w->L.n_out)
    return fail(SBN_ERR_INVALID_ARG, "%s: ld_y=%lld < n_out=%lld", name, (long long)ld_y,
                (long long)w->L.n_out);
  if (T == 0) return SBN_OK;
  if (!x_bf16 || !x_q || !x_absmax || (!y && w->L.n_out > 0))
    return fail(SBN_ERR_INVALID_ARG, "%s: null pointer", name);
  const_cast<sbn_packed*>(w)->last_stream = (hipStream_t)stream;
  // (the outlier term, if any, is added inside: in the same launch for one token)
  hipError_t e = sbn::launch_bitlinear_bf16(w, x_bf16, ld_x, T, x_q, ld_q, x_absmax, y, ld_y,
                                            (int)out_kind, ln_eps, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, name);
  return SBN_OK;
}

// The int8-input forward of one weight (the dispatch of sbn_bitlinear_fwd after validation).
hipError_t fwd_int8(const sbn_packed* w, const int8_t* x_q, int64_t ld_q, const float* x_absmax,
                    int64_t T, void* y, int64_t ld_y, sbn_out_kind out_kind, hipStream_t s) {
  if (w->L.n_out == 0) return hipSuccess;
  const_cast<sbn_packed*>(w)->last_stream = s;
  if (out_kind == SBN_OUT_F32 && sbn::gemv_int8_outl_fits(w, x_q, T))
    return sbn::launch_gemv_int8_outl(w, x_q, x_absmax, static_cast<float*>(y), s);
  hipError_t e = sbn::launch_bitlinear(w, x_q, ld_q, x_absmax, T, y, ld_y, (int)out_kind, s);
  if (e == hipSuccess && w->outlier_k > 0 && out_kind == SBN_OUT_F32)
    e = sbn::launch_outlier_add(w, x_q, ld_q, x_absmax, T, static_cast<float*>(y), ld_y, s);
  return e;
}

// Shared validation of the grouped forwards; ok_single is set when one grouped launch can serve
// them (same pattern and code form, no compact plane, no outlier term in the output, every member
// with rows).
sbn_status check_group(const char* name, const sbn_packed* const* ws, int count, int64_t T,
                       int64_t ld_q, void* const* ys, const int64_t* ld_ys, sbn_out_kind out_kind,
                       bool& ok_single) {
  if (!ws || !ys || !ld_ys) return fail(SBN_ERR_INVALID_ARG, "%s: null host array", name);
  if (count < 1 || count > SBN_MAX_GROUP)
    return fail(SBN_ERR_INVALID_ARG, "%s: count=%d outside [1, %d]", name, count, SBN_MAX_GROUP);
  if (out_kind != SBN_OUT_F32 && out_kind != SBN_OUT_I32_ACC)
    return fail(SBN_ERR_INVALID_ARG, "%s: out_kind=%d", name, (int)out_kind);
  if (T < 0) return fail(SBN_ERR_INVALID_ARG, "%s: T=%lld < 0", name, (long long)T);
  if (T > INT32_MAX) return fail(SBN_ERR_UNSUPPORTED, "%s: T too large", name);
  for (int i = 0; i < count; ++i)
    if (!ws[i]) return fail(SBN_ERR_INVALID_ARG, "%s: ws[%d] is null", name, i);
  const sbn_packed* w0 = ws[0];
  ok_single = true;
  for (int i = 0; i < count; ++i) {
    const sbn_packed* w = ws[i];
    if (w->L.K != w0->L.K)
      return fail(SBN_ERR_SHAPE, "%s: ws[%d] has K=%lld, ws[0] K=%lld", name, i,
                  (long long)w->L.K, (long long)w0->L.K);
    if (ld_ys[i] < w->L.n_out)
      return fail(SBN_ERR_INVALID_ARG, "%s: ld_ys[%d]=%lld < n_out=%lld", name, i,
                  (long long)ld_ys[i], (long long)w->L.n_out);
    if (T > 0 && w->L.n_out > 0 && !ys[i])
      return fail(SBN_ERR_INVALID_ARG, "%s: ys[%d] is null", name, i);
    if (w->L.n != w0->L.n || w->L.m != w0->L.m || w->L.form != w0->L.form || w->compact ||
        (w->outlier_k > 0 && out_kind == SBN_OUT_F32) || w->L.n_out == 0)
      ok_single = false;
  }
  if (ld_q < w0->L.K)
    return fail(SBN_ERR_INVALID_ARG, "%s: ld_q=%lld < K=%lld", name, (long long)ld_q,
                (long long)w0->L.K);
  if (ld_q > kMaxLdQ)
    return fail(SBN_ERR_UNSUPPORTED, "%s: ld_q=%lld > %lld", name, (long long)ld_q,
                (long long)kMaxLdQ);
  return SBN_OK;
}

}  // namespace

extern "C" {

const char* sbn_last_error(void) { return g_last_error; }

sbn_status sbn_bitlinear_fwd_group(const sbn_packed* const* ws, int count, const int8_t* x_q,
                                   int64_t ld_q, const float* x_absmax, int64_t T,
                                   void* const* ys, const int64_t* ld_ys, sbn_out_kind out_kind,
                                   void* stream) {
  const char* name = "sbn_bitlinear_fwd_group";
  bool single = false;
  sbn_status st = check_group(name, ws, count, T, ld_q, ys, ld_ys, out_kind, single);
  if (st != SBN_OK) return st;
  if (T == 0) return SBN_OK;
  if (!x_q || (out_kind == SBN_OUT_F32 && !x_absmax))
    return fail(SBN_ERR_INVALID_ARG, "%s: null pointer", name);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (single && T <= 16) {
    for (int i = 0; i < count; ++i) const_cast<sbn_packed*>(ws[i])->last_stream = s;
    e = sbn::launch_gemv_int8_group(ws, count, x_q, ld_q, x_absmax, T, ys, ld_ys, (int)out_kind, s);
  } else {
    for (int i = 0; i < count && e == hipSuccess; ++i)
      e = fwd_int8(ws[i], x_q, ld_q, x_absmax, T, ys[i], ld_ys[i], out_kind, s);
  }
  if (e != hipSuccess) return hip_fail(e, name);
  return SBN_OK;
}

sbn_status sbn_bitlinear_fwd_group_bf16(const sbn_packed* const* ws, int count,
                                        const uint16_t* x_bf16, int64_t ld_x, int64_t T,
                                        float ln_eps, int8_t* x_q, int64_t ld_q, float* x_absmax,
                                        void* const* ys, const int64_t* ld_ys,
                                        sbn_out_kind out_kind, void* stream) {
  const char* name = "sbn_bitlinear_fwd_group_bf16";
  bool single = false;
  sbn_status st = check_group(name, ws, count, T, ld_q, ys, ld_ys, out_kind, single);
  if (st != SBN_OK) return st;
  if (ld_x < ws[0]->L.K)
    return fail(SBN_ERR_INVALID_ARG, "%s: ld_x=%lld < K=%lld", name, (long long)ld_x,
                (long long)ws[0]->L.K);
  if (!(ln_eps >= 0.0f) || ln_eps > 3.0e38f)
    return fail(SBN_ERR_INVALID_ARG, "%s: ln_eps=%g must be 0 or positive and finite", name,
                (double)ln_eps);
  if (T == 0) return SBN_OK;
  if (!x_bf16 || !x_q || !x_absmax) return fail(SBN_ERR_INVALID_ARG, "%s: null pointer", name);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (single && sbn::gemv_group_fused_fits(ws[0], x_bf16, ld_x, T)) {
    for (int i = 0; i < count; ++i) const_cast<sbn_packed*>(ws[i])->last_stream = s;
    e = sbn::launch_gemv_group_bf16(ws, count, x_bf16, ld_x, T, x_q, ld_q, x_absmax, ys, ld_ys,
                                    (int)out_kind, ln_eps, s);
  } else {
    // the first member quantizes (one kernel where it can), the others read its x_q and a'
    const_cast<sbn_packed*>(ws[0])->last_stream = s;
    e = sbn::launch_bitlinear_bf16(ws[0], x_bf16, ld_x, T, x_q, ld_q, x_absmax, ys[0], ld_ys[0],
                                   (int)out_kind, ln_eps, s);
    for (int i = 1; i < count && e == hipSuccess; ++i)
      e = fwd_int8(ws[i], x_q, ld_q, x_absmax, T, ys[i], ld_ys[i], out_kind, s);
  }
  if (e != hipSuccess) return hip_fail(e, name);
  return SBN_OK;
}

sbn_status sbn_quantize_act(const uint16_t* x_bf16, int64_t T, int64_t K, int64_t ld_x,
                            int8_t* x_q, int64_t ld_q, float* x_absmax, void* stream) {
  if (T < 0) return fail(SBN_ERR_INVALID_ARG, "sbn_quantize_act: T=%lld < 0", (long long)T);
  if (K < 1 || K > SBN_MAX_K)
    return fail(SBN_ERR_INVALID_ARG, "sbn_quantize_act: K=%lld outside [1, %d]", (long long)K,
                SBN_MAX_K);
  if (ld_x < K || ld_q < K)
    return fail(SBN_ERR_INVALID_ARG, "sbn_quantize_act: ld_x=%lld / ld_q=%lld < K=%lld",
                (long long)ld_x, (long long)ld_q, (long long)K);
  if (T > INT32_MAX) return fail(SBN_ERR_UNSUPPORTED, "sbn_quantize_act: T too large");
  if (T == 0) return SBN_OK;
  if (!x_bf16 || !x_q || !x_absmax)
    return fail(SBN_ERR_INVALID_ARG, "sbn_quantize_act: null pointer");
  hipError_t e = sbn::launch_quantize_act(x_bf16, T, K, ld_x, x_q, ld_q, x_absmax,
                                          (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sbn_quantize_act launch");
  return SBN_OK;
}

sbn_status sbn_layernorm_quantize_act(const uint16_t* x_bf16, int64_t T, int64_t K,
                                      int64_t ld_x, float eps, int8_t* x_q, int64_t ld_q,
                                      float* x_absmax, void* stream) {
  if (T < 0)
    return fail(SBN_ERR_INVALID_ARG, "sbn_layernorm_quantize_act: T=%lld < 0", (long long)T);
  if (K < 1 || K > SBN_MAX_K)
    return fail(SBN_ERR_INVALID_ARG, "sbn_layernorm_quantize_act: K=%lld outside [1, %d]",
                (long long)K, SBN_MAX_K);
  if (ld_x < K || ld_q < K)
    return fail(SBN_ERR_INVALID_ARG, "sbn_layernorm_quantize_act: ld_x=%lld / ld_q=%lld < K",
                (long long)ld_x, (long long)ld_q);
  if (!(eps > 0.0f) || eps > 3.0e38f)
    return fail(SBN_ERR_INVALID_ARG, "sbn_layernorm_quantize_act: eps=%g must be > 0 and finite",
                (double)eps);
  if (T > INT32_MAX) return fail(SBN_ERR_UNSUPPORTED, "sbn_layernorm_quantize_act: T too large");
  if (T == 0) return SBN_OK;
  if (!x_bf16 || !x_q || !x_absmax)
    return fail(SBN_ERR_INVALID_ARG, "sbn_layernorm_quantize_act: null pointer");
  hipError_t e = sbn::launch_ln_quantize_act(x_bf16, T, K, ld_x, eps, x_q, ld_q, x_absmax,
                                             (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sbn_layernorm_quantize_act launch");
  return SBN_OK;
}

sbn_status sbn_pack_nm_ternary(const float* w_latent, int64_t n_out, int64_t K, int64_t ld_w,
                               int n_keep, int m_group, sbn_packed** handle, void* stream) {
  return sbn_pack_nm_ternary_ex(w_latent, n_out, K, ld_w, n_keep, m_group, 0, handle, stream);
}

sbn_status sbn_pack_nm_ternary_ex(const float* w_latent, int64_t n_out, int64_t K, int64_t ld_w,
                                  int n_keep, int m_group, int flags, sbn_packed** handle,
                                  void* stream) {
  if ((flags & ~(SBN_PACK_VARIANCE_CORRECTION | SBN_PACK_COMPACT | SBN_PACK_OUTLIERS(0xFF))) != 0)
    return fail(SBN_ERR_INVALID_ARG, "sbn_pack_nm_ternary: unknown flags 0x%x", flags);
  const int outlier_k = (flags >> 8) & 0xFF;
  if (outlier_k != 0 && outlier_k != 4 && outlier_k != 8 && outlier_k != 16)
    return fail(SBN_ERR_INVALID_ARG, "sbn_pack_nm_ternary: outliers per 256 must be 4, 8 or 16, not %d",
                outlier_k);
  if (outlier_k != 0 && K % 256 != 0)
    return fail(SBN_ERR_UNSUPPORTED, "sbn_pack_nm_ternary: k:256 outliers need K %% 256 == 0 (K=%lld)",
                (long long)K);
  if (!handle) return fail(SBN_ERR_INVALID_ARG, "sbn_pack_nm_ternary: handle is null");
  if (!pattern_ok(n_keep, m_group))
    return fail(SBN_ERR_UNSUPPORTED,
                "sbn_pack_nm_ternary: pattern %d:%d (need m in {4,8,16}, 1 <= n <= m)", n_keep,
                m_group);
  if (K < m_group || K > SBN_MAX_K || K % m_group != 0)
    return fail(SBN_ERR_INVALID_ARG,
                "sbn_pack_nm_ternary: K=%lld must be a multiple of m=%d in [m, %d]",
                (long long)K, m_group, SBN_MAX_K);
  if (n_out < 0 || n_out > INT32_MAX)
    return fail(SBN_ERR_INVALID_ARG, "sbn_pack_nm_ternary: n_out=%lld outside [0, 2^31)",
                (long long)n_out);
  if (ld_w < K)
    return fail(SBN_ERR_INVALID_ARG, "sbn_pack_nm_ternary: ld_w=%lld < K=%lld", (long long)ld_w,
                (long long)K);
  if (!w_latent && n_out > 0) return fail(SBN_ERR_INVALID_ARG, "sbn_pack_nm_ternary: w is null");

  sbn_packed* h = *handle;
  hipStream_t s = (hipStream_t)stream;
  if (h) {
    if (h->L.n_out != n_out || h->L.K != K || h->L.n != n_keep || h->L.m != m_group)
      return fail(SBN_ERR_SHAPE,
                  "sbn_pack_nm_ternary: handle is %lldx%lld %d:%d, call asks %lldx%lld %d:%d",
                  (long long)h->L.n_out, (long long)h->L.K, h->L.n, h->L.m, (long long)n_out,
                  (long long)K, n_keep, m_group);
  } else {
    sbn::Layout L;
    L.n_out = n_out;
    L.K = K;
    L.n = n_keep;
    L.m = m_group;
    L.positional = sbn::positional_codes(n_keep, m_group) ? 1 : 0;
    L.form = L.positional ? sbn::kFormPositional : sbn::kFormKept;
    // 2:4 uses the structured-sparse MFMA operands unless SBN_NO_SMFMAC is set to a non-zero
    // value (a diagnostic switch for comparing against the dense MFMA path).
    const char* no_sp = getenv("SBN_NO_SMFMAC");
    if (n_keep == 2 && m_group == 4 && !(no_sp && atoi(no_sp) != 0)) L.form = sbn::kFormSparse24;
    L.code_brick_bytes = L.positional ? 16 : 16 * n_keep / m_group;
    L.has_mask = n_keep < m_group ? 1 : 0;
    L.row_blocks = (n_out + 15) / 16;
    L.row_blocks_pad = (L.row_blocks + sbn::kPadRowBlocks - 1) / sbn::kPadRowBlocks *
                       sbn::kPadRowBlocks;
    L.quads = ((K + sbn::kBrickK - 1) / sbn::kBrickK + 3) / 4;
    L.csb = sbn::kBrickK * n_keep / m_group;
    if (16 * n_keep % m_group != 0)
      return fail(SBN_ERR_UNSUPPORTED, "sbn_pack_nm_ternary: pattern %d:%d", n_keep, m_group);
    const size_t slots = (size_t)L.row_blocks_pad * (size_t)L.quads * 64;
    const int num_partials = sbn::absmean_blocks(n_out);
    const size_t mask_bytes = L.has_mask ? slots * 8 : 0;
    const size_t code_bytes = slots * (size_t)L.code_brick_bytes;
    size_t off = 0;
    const size_t off_mask = off;
    off = align_up(off + mask_bytes, 256);
    const size_t off_codes = off;
    off = align_up(off + code_bytes, 256);
    const size_t off_gamma = off;
    off = align_up(off + sizeof(float), 256);
    const size_t off_part = off;
    off = align_up(off + sizeof(double) * num_partials, 256);
    const size_t off_sync = off;
    off = align_up(off + sizeof(int) * sbn::kGemmSyncInts, 256);
    const size_t off_flips = off;
    off = align_up(off + sizeof(uint32_t) * slots / 16, 256);  // 4 waves per fragment
    const size_t off_vc = off;
    off = align_up(off + 2 * sizeof(uint32_t) * slots / 16, 256);
    const size_t off_gamma_vc = off;
    off = align_up(off + sizeof(float), 256);
    const int64_t rq_count = (n_out + 127) / 128;
    const size_t off_tplane = off;
    off = align_up(off + (size_t)rq_count * (size_t)L.quads * 8192, 256);
    const size_t cplane_bytes =
        (size_t)L.row_blocks_pad * (size_t)L.quads * (size_t)sbn::compact_quad_bytes(L.csb) +
        sbn::kCompactSlack;
    const size_t off_cplane = off;
    off = align_up(off + cplane_bytes, 256);
    // structured-outlier planes (for up to 16 per 256 weights), when K is a multiple of 256
    const bool oplanes = K % 256 == 0;
    const size_t ogroups = oplanes ? (size_t)n_out * (size_t)(K / 256) : 0;
    const size_t off_opos = off;
    off = align_up(off + ogroups * 16, 256);
    const size_t off_oval = off;
    off = align_up(off + ogroups * 16 * sizeof(uint16_t), 256);
    const size_t off_omask = off;
    off = align_up(off + (oplanes ? slots * 8 : 0), 256);
    const size_t off_osum = off;
    off = align_up(off + ogroups * sizeof(double), 256);

    h = new (std::nothrow) sbn_packed;
    if (!h) return fail(SBN_ERR_OOM, "sbn_pack_nm_ternary: host allocation failed");
    h->L = L;
    h->code_row_bytes = (size_t)((K / m_group) * 2 * n_keep + 7) / 8;
    h->mask_row_bytes = L.has_mask ? (size_t)(K + 7) / 8 : 0;
    h->mask_plane_bytes = mask_bytes;
    h->code_plane_bytes = code_bytes;
    h->num_partials = num_partials;
    h->base_bytes = off;
    h->last_stream = s;
    hipError_t e = hipGetDevice(&h->device);
    if (e != hipSuccess) {
      delete h;
      return hip_fail(e, "sbn_pack_nm_ternary: hipGetDevice");
    }
    e = hipMalloc(&h->base, h->base_bytes);
    if (e != hipSuccess) {
      delete h;
      (void)hipGetLastError();
      return fail(SBN_ERR_OOM, "sbn_pack_nm_ternary: hipMalloc(%zu) failed", off);
    }
    // Padding bricks are never written by the pack kernel and must read as zero.
    e = hipMemsetAsync(h->base, 0, h->base_bytes, s);
    if (e != hipSuccess) {
      (void)hipFree(h->base);
      delete h;
      return hip_fail(e, "sbn_pack_nm_ternary: hipMemsetAsync");
    }
    h->mask = L.has_mask ? h->base + off_mask : nullptr;
    h->codes = h->base + off_codes;
    h->gamma = reinterpret_cast<float*>(h->base + off_gamma);
    h->partials = reinterpret_cast<double*>(h->base + off_part);
    h->gemm_sync = reinterpret_cast<int*>(h->base + off_sync);
    h->flip_parts = reinterpret_cast<uint32_t*>(h->base + off_flips);
    h->vc_parts = reinterpret_cast<uint32_t*>(h->base + off_vc);
    h->gamma_vc = reinterpret_cast<float*>(h->base + off_gamma_vc);
    h->vc = false;
    h->tplane = reinterpret_cast<uint32_t*>(h->base + off_tplane);
    h->rq_count = rq_count;
    h->cplane = h->base + off_cplane;
    h->cplane_bytes = cplane_bytes;
    h->compact_row_bytes = (size_t)(((K / m_group) * (m_group + n_keep) + 7) / 8);
    h->compact = false;
    h->outlier_k = 0;
    h->outlier_planes = oplanes;
    h->opos = h->base + off_opos;
    h->oval = reinterpret_cast<uint16_t*>(h->base + off_oval);
    h->omask = reinterpret_cast<unsigned long long*>(h->base + off_omask);
    h->osum = reinterpret_cast<double*>(h->base + off_osum);
    *handle = h;
  }
  h->last_stream = s;
  h->tplane_valid = false;  // rebuilt from the new codes by the next data-gradient call
  h->vc = (flags & SBN_PACK_VARIANCE_CORRECTION) != 0;
  h->compact = (flags & SBN_PACK_COMPACT) != 0;
  h->outlier_k = outlier_k;
  hipError_t e = sbn::launch_pack(w_latent, ld_w, h, s);
  if (e != hipSuccess) return hip_fail(e, "sbn_pack_nm_ternary launch");
  return SBN_OK;
}

sbn_status sbn_bitlinear_fwd(const sbn_packed* w, const int8_t* x_q, int64_t ld_q,
                             const float* x_absmax, int64_t T, void* y, int64_t ld_y,
                             sbn_out_kind out_kind, void* stream) {
  if (!w) return fail(SBN_ERR_INVALID_ARG, "sbn_bitlinear_fwd: handle is null");
  if (out_kind != SBN_OUT_F32 && out_kind != SBN_OUT_I32_ACC)
    return fail(SBN_ERR_INVALID_ARG, "sbn_bitlinear_fwd: out_kind=%d", (int)out_kind);
  if (T < 0) return fail(SBN_ERR_INVALID_ARG, "sbn_bitlinear_fwd: T=%lld < 0", (long long)T);
  if (T > INT32_MAX) return fail(SBN_ERR_UNSUPPORTED, "sbn_bitlinear_fwd: T too large");
  if (ld_q < w->L.K)
    return fail(SBN_ERR_INVALID_ARG, "sbn_bitlinear_fwd: ld_q=%lld < K=%lld", (long long)ld_q,
                (long long)w->L.K);
  if (ld_q > kMaxLdQ)
    return fail(SBN_ERR_UNSUPPORTED, "sbn_bitlinear_fwd: ld_q=%lld > %lld", (long long)ld_q,
                (long long)kMaxLdQ);
  if (ld_y < w->L.n_out)
    return fail(SBN_ERR_INVALID_ARG, "sbn_bitlinear_fwd: ld_y=%lld < n_out=%lld",
                (long long)ld_y, (long long)w->L.n_out);
  if (T == 0) return SBN_OK;
  if (w->L.n_out == 0) return SBN_OK;
  if (!x_q || !y || (out_kind == SBN_OUT_F32 && !x_absmax))
    return fail(SBN_ERR_INVALID_ARG, "sbn_bitlinear_fwd: null pointer");
  // (one token with outliers: the outlier term in the GEMV's launch)
  hipError_t e = fwd_int8(w, x_q, ld_q, x_absmax, T, y, ld_y, out_kind, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sbn_bitlinear_fwd launch");
  return SBN_OK;
}

sbn_status sbn_bitlinear_fwd_bf16(const sbn_packed* w, const uint16_t* x_bf16, int64_t ld_x,
                                  int64_t T, int8_t* x_q, int64_t ld_q, float* x_absmax, void* y,
                                  int64_t ld_y, sbn_out_kind out_kind, void* stream) {
  return fwd_bf16("sbn_bitlinear_fwd_bf16", w, x_bf16, ld_x, T, 0.0f, x_q, ld_q, x_absmax, y,
                  ld_y, out_kind, stream);
}

sbn_status sbn_bitlinear_fwd_ln_bf16(const sbn_packed* w, const uint16_t* x_bf16, int64_t ld_x,
                                     int64_t T, float eps, int8_t* x_q, int64_t ld_q,
                                     float* x_absmax, void* y, int64_t ld_y,
                                     sbn_out_kind out_kind, void* stream) {
  if (!(eps > 0.0f) || eps > 3.0e38f)
    return fail(SBN_ERR_INVALID_ARG, "sbn_bitlinear_fwd_ln_bf16: eps=%g must be > 0 and finite",
                (double)eps);
  return fwd_bf16("sbn_bitlinear_fwd_ln_bf16", w, x_bf16, ld_x, T, eps, x_q, ld_q, x_absmax, y,
                  ld_y, out_kind, stream);
}

void sbn_free(sbn_packed* handle) {
  if (!handle) return;
  (void)hipStreamSynchronize(handle->last_stream);
  (void)hipFree(handle->base);
  delete handle;
}

sbn_status sbn_packed_export(const sbn_packed* w, int8_t* codes, uint8_t* keep_mask, float* gamma,
                             void* stream) {
  if (!w) return fail(SBN_ERR_INVALID_ARG, "sbn_packed_export: handle is null");
  hipError_t e = sbn::launch_export(w, codes, keep_mask, gamma, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sbn_packed_export launch");
  return SBN_OK;
}

sbn_status sbn_packed_export_rpf(const sbn_packed* w, uint8_t* code_bytes, uint8_t* mask_bytes,
                                 void* stream) {
  if (!w) return fail(SBN_ERR_INVALID_ARG, "sbn_packed_export_rpf: handle is null");
  hipError_t e = sbn::launch_export_rpf(w, code_bytes, mask_bytes, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sbn_packed_export_rpf launch");
  return SBN_OK;
}

sbn_status sbn_bitlinear_bwd_dx(const sbn_packed* w, const uint16_t* dy_bf16, int64_t ld_dy,
                                int64_t T, float* dx, int64_t ld_dx, void* stream) {
  if (!w) return fail(SBN_ERR_INVALID_ARG, "sbn_bitlinear_bwd_dx: handle is null");
  if (T < 0) return fail(SBN_ERR_INVALID_ARG, "sbn_bitlinear_bwd_dx: T=%lld < 0", (long long)T);
  if (T > INT32_MAX) return fail(SBN_ERR_UNSUPPORTED, "sbn_bitlinear_bwd_dx: T too large");
  if (ld_dy < w->L.n_out)
    return fail(SBN_ERR_INVALID_ARG, "sbn_bitlinear_bwd_dx: ld_dy=%lld < n_out=%lld",
                (long long)ld_dy, (long long)w->L.n_out);
  if (ld_dy > kMaxLdQ / 2)
    return fail(SBN_ERR_UNSUPPORTED, "sbn_bitlinear_bwd_dx: ld_dy=%lld > %lld", (long long)ld_dy,
                (long long)(kMaxLdQ / 2));
  if (ld_dx < w->L.K)
    return fail(SBN_ERR_INVALID_ARG, "sbn_bitlinear_bwd_dx: ld_dx=%lld < K=%lld",
                (long long)ld_dx, (long long)w->L.K);
  if (w->rq_count > (1 << 20))
    return fail(SBN_ERR_UNSUPPORTED, "sbn_bitlinear_bwd_dx: n_out=%lld too large",
                (long long)w->L.n_out);
  if (w->outlier_k > 0)
    return fail(SBN_ERR_UNSUPPORTED,
                "sbn_bitlinear_bwd_dx: the last pack kept k:256 outliers (forward only)");
  if (T == 0) return SBN_OK;
  if (!dx || (!dy_bf16 && w->L.n_out > 0))
    return fail(SBN_ERR_INVALID_ARG, "sbn_bitlinear_bwd_dx: null pointer");
  sbn_packed* h = const_cast<sbn_packed*>(w);
  h->last_stream = (hipStream_t)stream;
  hipError_t e = sbn::launch_bwd_dx(h, dy_bf16, ld_dy, T, dx, ld_dx, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sbn_bitlinear_bwd_dx launch");
  return SBN_OK;
}

sbn_status sbn_packed_mask_flips(const sbn_packed* w, uint64_t* flips, void* stream) {
  if (!w || !flips) return fail(SBN_ERR_INVALID_ARG, "sbn_packed_mask_flips: null pointer");
  hipError_t e = sbn::launch_sum_flips(w, flips, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sbn_packed_mask_flips launch");
  return SBN_OK;
}

sbn_status sbn_packed_export_outliers(const sbn_packed* w, uint8_t* positions, uint16_t* values,
                                      void* stream) {
  if (!w) return fail(SBN_ERR_INVALID_ARG, "sbn_packed_export_outliers: handle is null");
  if (w->outlier_k == 0)
    return fail(SBN_ERR_INVALID_ARG,
                "sbn_packed_export_outliers: the last pack kept no outliers (SBN_PACK_OUTLIERS)");
  hipError_t e = sbn::launch_export_outliers(w, positions, values, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sbn_packed_export_outliers launch");
  return SBN_OK;
}

sbn_status sbn_packed_export_compact(const sbn_packed* w, uint8_t* bytes, void* stream) {
  if (!w) return fail(SBN_ERR_INVALID_ARG, "sbn_packed_export_compact: handle is null");
  if (!w->compact)
    return fail(SBN_ERR_INVALID_ARG,
                "sbn_packed_export_compact: the last pack did not write the compact form "
                "(SBN_PACK_COMPACT)");
  if (!bytes && w->L.n_out > 0)
    return fail(SBN_ERR_INVALID_ARG, "sbn_packed_export_compact: bytes is null");
  hipError_t e = sbn::launch_export_compact(w, bytes, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sbn_packed_export_compact launch");
  return SBN_OK;
}

sbn_status sbn_packed_export_rank(const sbn_packed* w, uint8_t* bytes, void* stream) {
  if (!w) return fail(SBN_ERR_INVALID_ARG, "sbn_packed_export_rank: handle is null");
  if (!bytes && w->L.n_out > 0)
    return fail(SBN_ERR_INVALID_ARG, "sbn_packed_export_rank: bytes is null");
  hipError_t e = sbn::launch_export_rank(w, bytes, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sbn_packed_export_rank launch");
  return SBN_OK;
}

sbn_status sbn_packed_query(const sbn_packed* w, sbn_packed_desc* out) {
  if (!w || !out) return fail(SBN_ERR_INVALID_ARG, "sbn_packed_query: null pointer");
  out->n_out = w->L.n_out;
  out->K = w->L.K;
  out->n = w->L.n;
  out->m = w->L.m;
  out->code_row_bytes = w->code_row_bytes;
  out->mask_row_bytes = w->mask_row_bytes;
  out->rpf_bytes = (size_t)w->L.n_out * (w->code_row_bytes + w->mask_row_bytes);
  out->packed_bytes = w->L.positional ? w->code_plane_bytes
                                      : w->mask_plane_bytes + w->code_plane_bytes;
  out->device_bytes = w->base_bytes;
  out->compact_row_bytes = w->compact_row_bytes;
  out->compact_bytes = w->cplane_bytes - sbn::kCompactSlack;
  out->compact = w->compact ? 1 : 0;
  out->outlier_k = w->outlier_k;
  out->rank_row_bytes =
      (size_t)(((w->L.K / w->L.m) * (sbn::rank_bits((int)w->L.n, (int)w->L.m) + 2 * w->L.n) + 7) /
               8);
  return SBN_OK;
}

}  // extern "C"
