// The dynamic-sparsity forward from the latent weights with no device allocation: the pack of
// sbn_pack_nm_ternary followed by sbn_bitlinear_fwd, with the packed planes, the absmean partial
// sums and the split-K words in a fixed device array of this library instead of a handle's
// allocation. For callers that cannot allocate (code under HIP graph capture, serving loops,
// harnesses that forbid allocation). Declared in include/sbn.h.
#include <algorithm>
#include <mutex>

#include "sbn_internal.hpp"

namespace sbn {
namespace {
constexpr size_t kStaticBytes = SBN_STATIC_WORKSPACE_BYTES;
}  // namespace
}  // namespace sbn

// The workspace. Each device the library runs on holds its own copy until the process ends. Host
// code reaches it only through the address hipGetSymbolAddress returns on that device (the array's
// name is a host-side stand-in there).
static __device__ __align__(256) uint8_t scratch[sbn::kStaticBytes];

namespace sbn {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
uint8_t* g_scratch[kMaxDevices];  // per device, set once

hipError_t scratch_on_current_device(uint8_t*& out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = static_cast<uint8_t*>(p);
  }
  out = g_scratch[dev];
  return hipSuccess;
}

// Zeroes n16 16-byte words (a fill kernel, not a memset: it may sit in a captured graph).
__global__ __launch_bounds__(256) void fill_zero(uint4* __restrict__ p, uint64_t n16) {
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_fill_zero(uint8_t* p, size_t bytes, hipStream_t s) {
  const uint64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<uint64_t>(2048, (n16 + 255) / 256);
  hipLaunchKernelGGL(fill_zero, dim3(blocks), dim3(256), 0, s, reinterpret_cast<uint4*>(p), n16);
  return hipGetLastError();
}

}  // namespace
}  // namespace sbn

extern "C" sbn_status sbn_bitlinear_fwd_latent_static(
    const float* w_latent, int64_t n_out, int64_t K, int64_t ld_w, int n_keep, int m_group,
    const int8_t* x_q, int64_t ld_q, const float* x_absmax, int64_t T, void* y, int64_t ld_y,
    sbn_out_kind out_kind, void* stream) {
  const char* name = "sbn_bitlinear_fwd_latent_static";
  if ((m_group != 4 && m_group != 8 && m_group != 16) || n_keep < 1 || n_keep > m_group)
    return sbn::set_error(SBN_ERR_UNSUPPORTED, "%s: pattern %d:%d (need m in {4,8,16}, 1 <= n <= m)",
                          name, n_keep, m_group);
  if (K < m_group || K > SBN_MAX_K || K % m_group != 0)
    return sbn::set_error(SBN_ERR_INVALID_ARG, "%s: K=%lld must be a multiple of m=%d in [m, %d]",
                          name, (long long)K, m_group, SBN_MAX_K);
  if (n_out < 0 || n_out > INT32_MAX)
    return sbn::set_error(SBN_ERR_INVALID_ARG, "%s: n_out=%lld outside [0, 2^31)", name,
                          (long long)n_out);
  if (ld_w < K)
    return sbn::set_error(SBN_ERR_INVALID_ARG, "%s: ld_w=%lld < K=%lld", name, (long long)ld_w,
                          (long long)K);
  if (out_kind != SBN_OUT_F32 && out_kind != SBN_OUT_I32_ACC)
    return sbn::set_error(SBN_ERR_INVALID_ARG, "%s: out_kind=%d", name, (int)out_kind);
  if (T < 0) return sbn::set_error(SBN_ERR_INVALID_ARG, "%s: T=%lld < 0", name, (long long)T);
  if (T > INT32_MAX) return sbn::set_error(SBN_ERR_UNSUPPORTED, "%s: T too large", name);
  if (ld_q < K || ld_q > ((int64_t)1 << 26))
    return sbn::set_error(SBN_ERR_INVALID_ARG, "%s: ld_q=%lld outside [K, 2^26]", name,
                          (long long)ld_q);
  if (ld_y < n_out)
    return sbn::set_error(SBN_ERR_INVALID_ARG, "%s: ld_y=%lld < n_out=%lld", name,
                          (long long)ld_y, (long long)n_out);
  sbn::Plan p;
  sbn_status st = sbn::make_plan(n_out, K, n_keep, m_group, p);
  if (st != SBN_OK) return st;
  if (p.forward_bytes > sbn::kStaticBytes)
    return sbn::set_error(SBN_ERR_UNSUPPORTED,
                          "%s: a %lldx%lld %d:%d weight needs %zu bytes of workspace, more than the "
                          "%zu this entry holds",
                          name, (long long)n_out, (long long)K, n_keep, m_group, p.forward_bytes,
                          sbn::kStaticBytes);
  if (T == 0 || n_out == 0) return SBN_OK;
  if (!w_latent || !x_q || !y || (out_kind == SBN_OUT_F32 && !x_absmax))
    return sbn::set_error(SBN_ERR_INVALID_ARG, "%s: null pointer", name);
  uint8_t* base = nullptr;
  hipError_t e = sbn::scratch_on_current_device(base);
  if (e != hipSuccess)
    return sbn::set_error(SBN_ERR_HIP, "%s: workspace address: %s", name, hipGetErrorString(e));
  hipStream_t s = (hipStream_t)stream;
  // A handle on the stack whose planes point into the workspace (plain values: no allocation).
  sbn_packed h{};
  sbn::bind_planes(h, p, base);
  sbn::splitk_settings(h.splitk_spin_limit, h.splitk_publish);
  h.base_bytes = p.forward_bytes;
  // the regions past forward_bytes (data-gradient, compact and outlier planes) do not exist here
  h.tplane = nullptr;
  h.cplane = nullptr;
  h.cplane_bytes = 0;
  h.outlier_planes = false;
  h.opos = nullptr;
  h.oval = nullptr;
  h.omask = nullptr;
  h.osum = nullptr;
  h.band_part = nullptr;  // a fresh handle: the two-pass pack
  h.band_seg = nullptr;
  h.band_lim = nullptr;
  h.band_slots = nullptr;
  h.gamma_valid = false;
  h.last_stream = s;
  // The planes' padding bricks must read as zero and the split-K words start at zero; the
  // workspace holds whatever the last call on this device left.
  e = sbn::launch_fill_zero(base, p.off_gamma, s);
  if (e == hipSuccess) e = sbn::launch_fill_zero(base + p.off_sync, p.off_flips - p.off_sync, s);
  if (e == hipSuccess) e = sbn::launch_pack(w_latent, ld_w, &h, s);
  if (e == hipSuccess)
    e = sbn::launch_bitlinear(&h, x_q, ld_q, x_absmax, T, y, ld_y, (int)out_kind, s);
  if (e != hipSuccess) return sbn::set_error(SBN_ERR_HIP, "%s launch: %s", name, hipGetErrorString(e));
  return SBN_OK;
}
