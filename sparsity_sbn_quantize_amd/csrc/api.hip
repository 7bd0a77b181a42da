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

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

sbn_status set_error(sbn_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

sbn_status make_plan(int64_t n_out, int64_t K, int n, int m, Plan& p) {
  Layout& L = p.L;
  L.n_out = n_out;
  L.K = K;
  L.n = n;
  L.m = m;
  L.positional = positional_codes(n, m) ? 1 : 0;
  L.form = L.positional ? kFormPositional : kFormKept;
  // 2:4 uses the structured-sparse MFMA operands unless SBN_NO_SMFMAC is set to a non-zero value
  // (a diagnostic switch for comparing against the dense MFMA path).
  const char* no_sp = getenv("SBN_NO_SMFMAC");
  if (n == 2 && m == 4 && !(no_sp && atoi(no_sp) != 0)) L.form = kFormSparse24;
  L.code_brick_bytes = L.positional ? 16 : 16 * n / m;
  L.has_mask = n < m ? 1 : 0;
  L.row_blocks = (n_out + 15) / 16;
  L.row_blocks_pad = (L.row_blocks + kPadRowBlocks - 1) / kPadRowBlocks * kPadRowBlocks;
  L.quads = ((K + kBrickK - 1) / kBrickK + 3) / 4;
  L.csb = kBrickK * n / m;
  if (16 * n % m != 0)
    return set_error(SBN_ERR_UNSUPPORTED, "sbn_pack_nm_ternary: pattern %d:%d", n, m);
  const size_t slots = (size_t)L.row_blocks_pad * (size_t)L.quads * 64;
  p.num_partials = absmean_blocks(n_out);
  p.mask_bytes = L.has_mask ? slots * 8 : 0;
  p.code_bytes = slots * (size_t)L.code_brick_bytes;
  size_t off = 0;
  p.off_mask = off;
  off = align_up(off + p.mask_bytes, 256);
  p.off_codes = off;
  off = align_up(off + p.code_bytes, 256);
  p.off_gamma = off;
  off = align_up(off + sizeof(float), 256);
  p.off_part = off;
  off = align_up(off + sizeof(double) * p.num_partials, 256);
  // large-K GEMV split over K: its counters follow the split-K words (zeroed together)
  const bool kx = L.quads >= kKxMinQuads && L.quads <= kKxMaxQuads && L.form != kFormKept;
  p.kx_chunks = kx ? (int)((L.quads + kKxQuads - 1) / kKxQuads) : 0;
  const int64_t kx_groups = kx ? kx_row_groups(L.row_blocks) : 0;
  p.off_sync = off;
  p.gen_index = kGemmSyncInts + 1 + (int)kx_groups;
  off = align_up(off + sizeof(uint32_t) * (p.gen_index + 2), 256);
  p.off_flips = off;
  off = align_up(off + sizeof(uint32_t) * slots / 16, 256);  // 4 waves per fragment
  p.off_vc = off;
  off = align_up(off + 2 * sizeof(uint32_t) * slots / 16, 256);
  p.off_gamma_vc = off;
  off = align_up(off + sizeof(float), 256);
  p.off_kx = off;
  off = align_up(off + (size_t)kx_groups * p.kx_chunks * 16 * 1024, 256);
  p.forward_bytes = off;  // everything the pack and the forward use
  p.rq_count = (n_out + 127) / 128;
  p.off_tplane = off;
  off = align_up(off + (size_t)p.rq_count * (size_t)L.quads * 8192, 256);
  p.cplane_bytes =
      (size_t)L.row_blocks_pad * (size_t)L.quads * (size_t)compact_quad_bytes(L.csb) +
      kCompactSlack;
  p.off_cplane = off;
  off = align_up(off + p.cplane_bytes, 256);
  // structured-outlier planes (for up to 16 per 256 weights), when K is a multiple of 256
  p.oplanes = K % 256 == 0;
  const size_t ogroups = p.oplanes ? (size_t)n_out * (size_t)(K / 256) : 0;
  p.off_opos = off;
  off = align_up(off + ogroups * 16, 256);
  p.off_oval = off;
  off = align_up(off + ogroups * 16 * sizeof(uint16_t), 256);
  p.off_omask = off;
  off = align_up(off + (p.oplanes ? slots * 8 : 0), 256);
  p.off_osum = off;
  off = align_up(off + ogroups * sizeof(double), 256);
  // single-pass re-pack: per-fragment partial sums, listed-piece counts and lists, the bracket
  const size_t frags = (size_t)L.row_blocks_pad * (size_t)L.quads;
  p.off_band = off;
  off = align_up(off + frags * (sizeof(double) + kBandRecBytes) + 512 + kBandSlots * 128, 256);
  p.total_bytes = off;
  return SBN_OK;
}

void bind_planes(sbn_packed& h, const Plan& p, uint8_t* base) {
  const Layout& L = p.L;
  h.L = L;
  h.code_row_bytes = (size_t)((L.K / L.m) * 2 * L.n + 7) / 8;
  h.mask_row_bytes = L.has_mask ? (size_t)(L.K + 7) / 8 : 0;
  h.mask_plane_bytes = p.mask_bytes;
  h.code_plane_bytes = p.code_bytes;
  h.num_partials = p.num_partials;
  h.base = base;
  h.base_bytes = p.total_bytes;
  h.mask = L.has_mask ? base + p.off_mask : nullptr;
  h.codes = base + p.off_codes;
  h.gamma = reinterpret_cast<float*>(base + p.off_gamma);
  h.partials = reinterpret_cast<double*>(base + p.off_part);
  h.gemm_sync = reinterpret_cast<uint32_t*>(base + p.off_sync);
  h.kx_count = h.gemm_sync + kGemmSyncInts + 1;
  h.pack_gen = h.gemm_sync + p.gen_index;
  h.kx_part = base + p.off_kx;
  h.kx_chunks = p.kx_chunks;
  h.flip_parts = reinterpret_cast<uint32_t*>(base + p.off_flips);
  h.vc_parts = reinterpret_cast<uint32_t*>(base + p.off_vc);
  h.gamma_vc = reinterpret_cast<float*>(base + p.off_gamma_vc);
  h.vc = false;
  h.tplane = reinterpret_cast<uint32_t*>(base + p.off_tplane);
  h.rq_count = p.rq_count;
  h.cplane = base + p.off_cplane;
  h.cplane_bytes = p.cplane_bytes;
  h.compact_row_bytes = (size_t)(((L.K / L.m) * (L.m + L.n) + 7) / 8);
  h.compact = false;
  h.outlier_k = 0;
  h.outlier_planes = p.oplanes;
  h.opos = base + p.off_opos;
  h.oval = reinterpret_cast<uint16_t*>(base + p.off_oval);
  h.omask = reinterpret_cast<unsigned long long*>(base + p.off_omask);
  h.osum = reinterpret_cast<double*>(base + p.off_osum);
  {
    const size_t frags = (size_t)L.row_blocks_pad * (size_t)L.quads;
    uint8_t* b = base + p.off_band;
    h.band_part = reinterpret_cast<double*>(b);
    h.band_seg = b + frags * sizeof(double);
    h.band_lim = reinterpret_cast<uint32_t*>(b + frags * (sizeof(double) + kBandRecBytes));
    h.band_slots = reinterpret_cast<unsigned long long*>(
        base + align_up(p.off_band + frags * (sizeof(double) + kBandRecBytes) + 256, 128));
  }
  h.gamma_valid = false;
  h.single_pass = false;
  h.splitk_spin_limit = kSplitSpinLimit;
  h.splitk_publish = 1;
}

void splitk_settings(int& spin_limit, int& publish) {
  // Test settings of the split-K handshake: SBN_SPLITK_SPIN_LIMIT (s_sleep rounds a waiting half
  // spins before it gives up) and SBN_SPLITK_WITHHOLD=1 (the first half never publishes, so every
  // waiting half gives up: exercises the give-up counter with every kernel exiting normally).
  spin_limit = kSplitSpinLimit;
  publish = 1;
  const char* lim = getenv("SBN_SPLITK_SPIN_LIMIT");
  if (lim && atoi(lim) > 0) spin_limit = atoi(lim);
  const char* wh = getenv("SBN_SPLITK_WITHHOLD");
  if (wh && atoi(wh) != 0) publish = 0;
}

}  // namespace sbn

namespace {

sbn_status hip_fail(hipError_t e, const char* what) {
  return fail(SBN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

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
  } else if (single && T <= 16) {
    // the quantizer, then the grouped int8 GEMV
    for (int i = 0; i < count; ++i) const_cast<sbn_packed*>(ws[i])->last_stream = s;
    e = ln_eps > 0.0f ? sbn::launch_ln_quantize_act(x_bf16, T, ws[0]->L.K, ld_x, ln_eps, x_q, ld_q,
                                                    x_absmax, s)
                      : sbn::launch_quantize_act(x_bf16, T, ws[0]->L.K, ld_x, x_q, ld_q, x_absmax,
                                                 s);
    if (e == hipSuccess)
      e = sbn::launch_gemv_int8_group(ws, count, x_q, ld_q, x_absmax, T, ys, ld_ys, (int)out_kind,
                                      s);
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
    sbn::Plan p;
    sbn_status st = sbn::make_plan(n_out, K, n_keep, m_group, p);
    if (st != SBN_OK) return st;
    h = new (std::nothrow) sbn_packed();
    if (!h) return fail(SBN_ERR_OOM, "sbn_pack_nm_ternary: host allocation failed");
    hipError_t e = hipGetDevice(&h->device);
    if (e != hipSuccess) {
      delete h;
      return hip_fail(e, "sbn_pack_nm_ternary: hipGetDevice");
    }
    // Stream-ordered allocation where the device has memory pools (released by sbn_free on the
    // handle's last stream without blocking the host); a plain allocation otherwise.
    int pools = 0;
    (void)hipDeviceGetAttribute(&pools, hipDeviceAttributeMemoryPoolsSupported, h->device);
    uint8_t* base = nullptr;
    h->async_alloc = pools != 0;
    e = h->async_alloc ? hipMallocAsync(reinterpret_cast<void**>(&base), p.total_bytes, s)
                       : hipMalloc(reinterpret_cast<void**>(&base), p.total_bytes);
    if (e != hipSuccess) {
      delete h;
      (void)hipGetLastError();
      return fail(SBN_ERR_OOM, "sbn_pack_nm_ternary: device allocation of %zu bytes failed",
                  p.total_bytes);
    }
    // Padding bricks are never written by the pack kernel and must read as zero; the split-K
    // words start at zero.
    e = hipMemsetAsync(base, 0, p.total_bytes, s);
    if (e != hipSuccess) {
      if (h->async_alloc) (void)hipFreeAsync(base, s); else (void)hipFree(base);
      delete h;
      return hip_fail(e, "sbn_pack_nm_ternary: hipMemsetAsync");
    }
    sbn::bind_planes(*h, p, base);
    *handle = h;
  }
  sbn::splitk_settings(h->splitk_spin_limit, h->splitk_publish);
  h->last_stream = s;
  h->vc = (flags & SBN_PACK_VARIANCE_CORRECTION) != 0;
  h->compact = (flags & SBN_PACK_COMPACT) != 0;
  h->outlier_k = outlier_k;
  hipError_t e = sbn::launch_pack(w_latent, ld_w, h, s);
  if (e != hipSuccess) return hip_fail(e, "sbn_pack_nm_ternary launch");
  h->gamma_valid = true;  // the next pack of this handle may bracket its threshold with gamma
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
  if (handle->async_alloc) {
    (void)hipFreeAsync(handle->base, handle->last_stream);
  } else {
    (void)hipStreamSynchronize(handle->last_stream);
    (void)hipFree(handle->base);
  }
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
  // the split-K give-up counter, read after the handle's last stream has drained
  uint32_t giveups = 0;
  hipError_t e = hipStreamSynchronize(w->last_stream);
  if (e == hipSuccess)
    e = hipMemcpy(&giveups, w->gemm_sync + sbn::kGemmSyncInts, sizeof(giveups),
                  hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "sbn_packed_query");
  out->splitk_giveups = giveups;
  out->single_pass = w->single_pass ? 1 : 0;
  return SBN_OK;
}

}  // extern "C"
