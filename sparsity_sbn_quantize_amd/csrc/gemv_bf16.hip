// One-token entry of the quantize-and-multiply GEMV ("Microsoft BitNet 1.58: The Era of 1-Bit
// Large Language Models", section "The BitLinear Layer": per-token absmax quantization, then the
// ternary matmul and the rescale, in one launch). The body is the bf16-input kernel's (gemv.hpp);
// this file is compiled with kernel-argument preloading, and the entry takes every value its first
// loads need (the activation row, the code plane, K, the quad count, the wave count, the scale and
// output pointers) in its first 16 argument dwords, with the wave count as an argument rather than
// the dispatch's group size, so the activation loads go out without waiting for a scalar load of
// the argument block.
#include "gemv.hpp"

namespace sbn {
namespace {

template <int FORM, int Q>
__global__ __launch_bounds__(kGemvMaxWaves * 64) void bitlinear_gemv_bf16_one(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ code_plane, int K, int nq, int W,
    int out_kind, const float* __restrict__ gamma_p, float* __restrict__ absmax,
    int8_t* __restrict__ xq_out, void* __restrict__ y, int64_t ld_q, int64_t ld_y,
    const uint8_t* __restrict__ mask_plane, Layout L) {
  gemv_body<FORM, true, true, Q, false, true>(mask_plane, code_plane, L, K, nq, W, gamma_p, x, 0,
                                              xq_out, ld_q, absmax, 1, y, ld_y, out_kind, 0.0f,
                                              (int64_t)blockIdx.x, blockIdx.x == 0);
}

template <int FORM>
hipError_t launch_one(const sbn_packed* h, const uint16_t* x, int8_t* xq, int64_t ld_q,
                      float* absmax, void* y, int64_t ld_y, int out_kind, hipStream_t s) {
  const Layout& L = h->L;
  // the wave and quad counts of the bf16 launcher (three quads per wave)
  const int W = (int)std::min<int64_t>(kGemvMaxWaves, (L.quads + kGemvMaxQ - 1) / kGemvMaxQ);
  const int Q = (int)((L.quads + W - 1) / W);
#define SBN_ONE(QQ)                                                                            \
  hipLaunchKernelGGL((bitlinear_gemv_bf16_one<FORM, QQ>), dim3((unsigned)L.row_blocks),         \
                     dim3(64 * W), 0, s, x, h->codes, (int)L.K, (int)L.quads, W, out_kind,       \
                     h->gamma_out(), absmax, xq, y, ld_q, ld_y, h->mask, L)
  if (Q == 1) {
    SBN_ONE(1);
  } else if (Q == 2) {
    SBN_ONE(2);
  } else {
    SBN_ONE(3);
  }
#undef SBN_ONE
  return hipGetLastError();
}

}  // namespace

bool gemv_bf16_one_fits(const sbn_packed* h, const uint16_t* x, int64_t T, float ln_eps) {
  const Layout& L = h->L;
  return T == 1 && ln_eps <= 0.0f && !h->compact && L.n_out > 0 && (uintptr_t)x % 8 == 0 &&
         L.K % 4 == 0 && L.quads <= (int64_t)kGemvMaxWaves * kGemvMaxQ;
}

hipError_t launch_gemv_bf16_one(const sbn_packed* h, const uint16_t* x, int8_t* xq, int64_t ld_q,
                                float* absmax, void* y, int64_t ld_y, int out_kind,
                                hipStream_t s) {
  if (h->L.form == kFormSparse24)
    return launch_one<kFormSparse24>(h, x, xq, ld_q, absmax, y, ld_y, out_kind, s);
  if (h->L.form == kFormPositional)
    return launch_one<kFormPositional>(h, x, xq, ld_q, absmax, y, ld_y, out_kind, s);
  return launch_one<kFormKept>(h, x, xq, ld_q, absmax, y, ld_y, out_kind, s);
}

}  // namespace sbn
