// Entry of the int8-input GEMV (T <= 16; "Microsoft BitNet 1.58: The Era of 1-Bit Large Language
// Models", section "The BitLinear Layer", operations 4 and 5). The kernel body is the one the
// bf16-input kernels use (gemv.hpp); this file is compiled with kernel-argument preloading, and
// its entry takes the values its first loads need (code plane, activations, quad count, K, leading
// dimension, token count, wave count, a', gamma) as leading scalar arguments, so those loads go out without waiting
// for a scalar load of the argument block (3.77 -> 3.57 us at T = 1 and 5.64 -> 5.35 us at T = 16
// on the 2560 -> 6912 shape). The bf16-input kernels keep their own argument order: moving their
// arguments the same way made them slower.
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
  const int blocks = make_group(hs, count, ys, ld_ys, G);
  const Layout& L = hs[0]->L;
  const bool xvec = ((uintptr_t)xq % 16 == 0) && (ld_q % 16 == 0) && (L.K % 16 == 0);
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
  if (xvec) return launch_i8_form<true>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
  return launch_i8_form<false>(h, xq, ld_q, absmax, T, y, ld_y, out_kind, s);
}

}  // namespace sbn
