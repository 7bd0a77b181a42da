/*
 * sbn.h - C ABI of the Sparse-BitNet BitLinear forward for AMD MI355X (gfx950).
 *
 * The forward of one BitLinear layer is split into three calls:
 *   sbn_quantize_act     per-token absmax INT8 activation quantization (sbn_layernorm_quantize_act
 *                        runs the layer's parameter-free LayerNorm first)
 *   sbn_pack_nm_ternary  per-tensor absmean ternary quantization of fp32 latent weights with a
 *                        dynamic n:m magnitude keep mask, packed as 2-bit codes + per-group mask
 *   sbn_bitlinear_fwd    n:m-sparse ternary x INT8 matmul, int32 accumulation, fused dequant
 * Sources: "Microsoft BitNet 1.58: The Era of 1-Bit Large Language Models", section "The BitLinear
 * Layer" (the five operations of BitLinear; latent full-precision weights re-quantized on every
 * forward) and section "bitnet.cpp: Matrix-Free Inference" (four 2-bit ternary values per byte,
 * integer dot products); "BitNet b1.58: How Ternary Weights Cut LLM Memory by 82% Without Losing
 * Accuracy", section "How ternary quantization works during training" (weights divided by their
 * mean absolute value, rounded, clamped to [-1, 1]; INT8 activations with a per-token scale);
 * "Sparse-BitNet: 1.58-bit LLMs are Naturally Friendly to Semi-Structured Sparsity", Abstract
 * (dynamic N:M sparsification applied jointly with 1.58-bit quantization), Figure 6 (the N largest
 * normalized magnitudes of each M-block are kept) and Table 6 (the N:8 patterns); "From 2:4 to
 * 8:16 sparsity patterns in LLMs for Outliers and Weights with Variance Correction", abstract
 * (the 8:16 pattern and its per-group index metadata).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked (host). Device memory belongs to the caller,
 *     except the packed-weight handle, which the library owns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Calls only enqueue
 *     work on it; none synchronizes the device (except sbn_packed_query and, on devices without
 *     memory pools, sbn_free; see there).
 *   - Arguments are validated on the host before any HIP call; a rejected call touches no GPU
 *     state and returns a negative sbn_status. sbn_last_error() then holds a message.
 *   - Shapes: T tokens, K input features (reduction axis), n_out output features. Leading
 *     dimensions (ld_*) are in elements and must be >= the row length.
 *   - NaN or Inf inputs give unspecified (but memory-safe) results.
 *   - The handle's device must be the current device for every call that uses it.
 *   - Calls that use one handle must be ordered (one stream, or synchronized by the caller): a
 *     forward that splits K over two workgroups per tile keeps its handshake words in the handle,
 *     and a re-pack rewrites the planes a forward reads.
 */
#ifndef SBN_H
#define SBN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SBN_OK = 0,
  SBN_ERR_INVALID_ARG = -1, /* null pointer, bad size, leading dimension or enum value */
  SBN_ERR_UNSUPPORTED = -2, /* pattern or size outside what the kernels implement */
  SBN_ERR_SHAPE = -3,       /* re-pack into a handle of another shape or pattern */
  SBN_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  SBN_ERR_OOM = -5          /* device allocation failed */
} sbn_status;

typedef enum {
  SBN_OUT_F32 = 0,    /* y fp32 = fl32(fl32(fl32(acc) * gamma) * fl32(a'_t / 127)) */
  SBN_OUT_I32_ACC = 1 /* y int32 = acc, the raw integer accumulator */
} sbn_out_kind;

/* Opaque packed ternary weight, owned by the library. */
typedef struct sbn_packed sbn_packed;

/* Upper bound on K: keeps every accumulator |acc| <= 127*K below 2^24, so fl32(acc) is exact. */
#define SBN_MAX_K (1 << 17)

/*
 * Per-token absmax INT8 activation quantization ("The BitLinear Layer", operation 2; per-token
 * scale in "How ternary quantization works during training").
 *   x_bf16    [T][ld_x] bf16 bit patterns (uint16), read only.
 *   x_q       [T][ld_q] int8 out: q = clamp(rne(fl32(x * s_t)), -127, 127),
 *             s_t = fl32(127 / a'_t) (correctly rounded fp32 division).
 *   x_absmax  [T] fp32 out: a'_t = max(max_k |x[t,k]|, 1e-5), the scale kept for dequantization.
 * Requires T >= 0, 1 <= K <= SBN_MAX_K, ld_x >= K, ld_q >= K; T == 0 is a no-op.
 * Columns K..ld-1 of x_q are not written.
 */
sbn_status sbn_quantize_act(const uint16_t* x_bf16, int64_t T, int64_t K, int64_t ld_x,
                            int8_t* x_q, int64_t ld_q, float* x_absmax, void* stream);

/*
 * Parameter-free LayerNorm followed by sbn_quantize_act ("The BitLinear Layer", operations 1 and
 * 2: activations are normalized without learned scale or shift, then quantized from BF16 to INT8).
 * The page gives no formula or epsilon; this is the standard LayerNorm without affine terms:
 *   mu = fl64(sum_k x[t,k] / K), var = fl64(sum_k (x - mu)^2 / K)  (biased; fp64 statistics)
 *   r  = fl64(1 / sqrt(var + eps))
 *   z[t,k] = bf16( fl32( fl32(x - fl32(mu)) * fl32(r) ) )           (round to nearest even)
 * and x_q, x_absmax are exactly what sbn_quantize_act writes for the bf16 rows z.
 *   x_bf16    [T][ld_x] bf16 bit patterns (uint16), read only.
 *   eps       > 0 and finite (1e-5 is the usual choice).
 * Requires T >= 0, 1 <= K <= SBN_MAX_K, ld_x >= K, ld_q >= K; T == 0 is a no-op.
 */
sbn_status sbn_layernorm_quantize_act(const uint16_t* x_bf16, int64_t T, int64_t K,
                                      int64_t ld_x, float eps, int8_t* x_q, int64_t ld_q,
                                      float* x_absmax, void* stream);

/*
 * Absmean ternary quantization with a dynamic n:m keep mask, packed ("The BitLinear Layer",
 * operation 3, with the divide reading of "How ternary quantization works during training";
 * Sparse-BitNet Abstract and Figure 6).
 *   w_latent  [n_out][ld_w] fp32 latent weights (nn.Linear layout), read only.
 *   gamma = fl32( sum|w| (fp64) / (n_out*K) ), one scale per tensor over the dense weights.
 *   keep: in each group of m consecutive weights along K of a row, the n largest |w|, equal
 *         magnitudes going to the lower position.
 *   code  = keep ? (|w| > gamma/2 ? sign(w) : 0) : 0   (= RoundClip(w/gamma, -1, 1), ties to even)
 *   *handle == NULL: a handle is allocated (stream-ordered on `stream` where the device has memory
 *   pools; with sbn_free, the only allocations the library makes) and returned in *handle (host). Otherwise the existing handle is re-packed in place, with no
 *   allocation; it must have been made with the same n_out, K, n_keep, m_group (else
 *   SBN_ERR_SHAPE). Every call recomputes gamma and the mask from the current weights.
 *   Reads of w_latent: the first pack of a handle reads it twice (gamma must be known before a
 *   code is written). A re-pack with flags 0 of the patterns 2:4, 4:8, 6:8, 8:16 and n = m reads
 *   it once: the previous gamma brackets the new threshold (gamma / 2 within 2^-7 of the old
 *   one), the few 16-weight pieces with a kept magnitude inside the bracket are finished after
 *   the new gamma is known, and if the threshold left the bracket the codes are rewritten from a
 *   second read. The planes are the same in every case; gamma is summed there in fixed point
 *   (2^50 units for the previous total, error below 2^-36 of the sum, so it rounds to the same
 *   fp32 value except that close to a rounding midpoint). sbn_packed_desc.single_pass says which
 *   path the last pack took.
 * Requires m_group in {4, 8, 16}, 1 <= n_keep <= m_group, K % m_group == 0,
 * m_group <= K <= SBN_MAX_K, 0 <= n_out < 2^31, ld_w >= K.
 */
sbn_status sbn_pack_nm_ternary(const float* w_latent, int64_t n_out, int64_t K, int64_t ld_w,
                               int n_keep, int m_group, sbn_packed** handle /* host */,
                               void* stream);

/* Flags of sbn_pack_nm_ternary_ex. */
#define SBN_PACK_VARIANCE_CORRECTION 1
#define SBN_PACK_COMPACT 2
#define SBN_PACK_OUTLIERS(k) ((k) << 8) /* k in {4, 8, 16}: k:256 structured outliers */

/*
 * sbn_pack_nm_ternary with options. SBN_PACK_VARIANCE_CORRECTION ("From 2:4 to 8:16 sparsity
 * patterns in LLMs for Outliers and Weights with Variance Correction", method summary: after
 * pruning, the remaining weights are rescaled back to the dense variance): the codes and the mask
 * are unchanged; the scale the matmuls use becomes gamma_out = fl32(gamma * sqrt(nd / ns)), with
 * nd the nonzero codes of the dense (n = m) ternary weights and ns those of the n:m codes
 * (gamma_out = gamma when ns == 0). The page gives no formula; this restores the mean square of
 * the ternary weights gamma * code, per tensor like gamma. sbn_bitlinear_fwd, the bf16 forwards,
 * sbn_bitlinear_bwd_dx and sbn_packed_export then use gamma_out.
 * SBN_PACK_COMPACT (inference encoding; "Why 1.58 Bits?" and "bitnet.cpp: Matrix-Free Inference"
 * in "Microsoft BitNet 1.58": a ternary weight holds log2 3 bits, packed weights are unpacked on
 * chip): the pack also writes a compact copy of the codes that keeps only which positions are
 * nonzero and their signs, (m + n) / m bits per weight (1.5 at 2:4 and 8:16, 1.75 at 6:8, against
 * 2 for the 2-bit codes), and every launch of the forwards with T <= 16 (the GEMV) reads it
 * instead of the 2-bit codes. Results are identical; sbn_packed_export_compact exports it.
 * SBN_PACK_OUTLIERS(k), k in {4, 8, 16} ("From 2:4 to 8:16 sparsity patterns ...", summary:
 * salient weights kept in structured k:256 patterns): in each group of 256 weights along K, the k
 * of largest |w| (equal magnitudes: the lower position) are kept apart as bf16 values (round to
 * nearest even); gamma, the keep mask, the codes and the variance-correction counts then use the
 * other weights, with the outlier positions read as 0. The fp32 forwards add the outlier term:
 * y = fl32(y_ternary + fl32(o * fl32(a'/127))), o = the fp32 sum, in a fixed order, of
 * x_q[t][position] * value over the row's outliers (each product is exact); the order is the same
 * on every path, so sbn_bitlinear_fwd and sbn_bitlinear_fwd_bf16 give the same bits. For one
 * token, n_out a multiple of 16, K <= 12288 and no SBN_PACK_COMPACT (and, for the bf16 entry, no
 * LayerNorm), both forwards add the term in the GEMV's launch; otherwise a second launch adds it. SBN_OUT_I32_ACC
 * returns the ternary accumulators only; sbn_bitlinear_bwd_dx rejects such a handle
 * (SBN_ERR_UNSUPPORTED: outliers are a post-training, inference-only variant). Needs
 * K % 256 == 0 (else SBN_ERR_UNSUPPORTED).
 * Each call may change the flags. flags = 0 is sbn_pack_nm_ternary; other bits give
 * SBN_ERR_INVALID_ARG.
 */
sbn_status sbn_pack_nm_ternary_ex(const float* w_latent, int64_t n_out, int64_t K, int64_t ld_w,
                                  int n_keep, int m_group, int flags, sbn_packed** handle /* host */,
                                  void* stream);

/*
 * n:m-sparse ternary x INT8 matmul with int32 accumulation and fused dequantization
 * ("The BitLinear Layer", operations 4 and 5).
 *   x_q       [T][ld_q] int8 (from sbn_quantize_act), x_absmax [T] fp32 (a'_t).
 *   acc[t][r] = sum_k x_q[t][k] * code[r][k]   (exact int32)
 *   y         [T][ld_y] fp32 (SBN_OUT_F32) or int32 (SBN_OUT_I32_ACC); x_absmax may be NULL
 *             for SBN_OUT_I32_ACC.
 * Requires T >= 0, K <= ld_q <= 2^26, ld_y >= n_out; T == 0 or n_out == 0 is a no-op.
 */
sbn_status sbn_bitlinear_fwd(const sbn_packed* w, const int8_t* x_q, int64_t ld_q,
                             const float* x_absmax, int64_t T, void* y, int64_t ld_y,
                             sbn_out_kind out_kind, void* stream);

/*
 * Quantize-and-multiply in one call: the per-token absmax INT8 quantization of sbn_quantize_act
 * followed by sbn_bitlinear_fwd ("The BitLinear Layer", operations 2, 4 and 5).
 *   x_bf16    [T][ld_x] bf16 bit patterns (uint16), read only.
 *   x_q       [T][ld_q] int8 out and x_absmax [T] fp32 out: exactly what sbn_quantize_act writes.
 *   y         [T][ld_y] as for sbn_bitlinear_fwd.
 * For T <= 4 and K <= 12288 the whole call is one kernel launch, in which every workgroup
 * quantizes the activations it needs itself; otherwise it runs the two kernels in turn.
 * Requires T >= 0, ld_x >= K, K <= ld_q <= 2^26, ld_y >= n_out; T == 0 is a no-op; y may be
 * NULL when n_out == 0 (x_q and x_absmax are still written).
 */
sbn_status sbn_bitlinear_fwd_bf16(const sbn_packed* w, const uint16_t* x_bf16, int64_t ld_x,
                                  int64_t T, int8_t* x_q, int64_t ld_q, float* x_absmax, void* y,
                                  int64_t ld_y, sbn_out_kind out_kind, void* stream);

/*
 * The whole BitLinear forward on bf16 input: sbn_layernorm_quantize_act then sbn_bitlinear_fwd
 * ("The BitLinear Layer", operations 1, 2, 4 and 5). x_q and x_absmax receive exactly what
 * sbn_layernorm_quantize_act writes; y is as for sbn_bitlinear_fwd. For T <= 4 and K <= 12288
 * the whole call is one kernel launch in which every workgroup normalizes and quantizes the rows
 * it needs itself; otherwise it runs the two kernels in turn. Requirements as for
 * sbn_bitlinear_fwd_bf16, with eps > 0 and finite.
 */
sbn_status sbn_bitlinear_fwd_ln_bf16(const sbn_packed* w, const uint16_t* x_bf16, int64_t ld_x,
                                     int64_t T, float eps, int8_t* x_q, int64_t ld_q,
                                     float* x_absmax, void* y, int64_t ld_y,
                                     sbn_out_kind out_kind, void* stream);

/* Most weights one grouped call takes. */
#define SBN_MAX_GROUP 8

/*
 * Grouped forward: several packed weights that read the same activations, for instance the Q, K
 * and V projections of a block, or its gate and up projections ("The BitLinear Layer", operations
 * 4 and 5, for each weight). The result is exactly that of sbn_bitlinear_fwd on each member in
 * turn with the same x_q and x_absmax:
 *   ws        [count] (host) packed weights, all with the same K (else SBN_ERR_SHAPE);
 *             1 <= count <= SBN_MAX_GROUP; a handle may appear more than once.
 *   ys        [count] (host) output pointers, member i's y [T][ld_ys[i]] as for sbn_bitlinear_fwd.
 *   ld_ys     [count] (host) leading dimensions, ld_ys[i] >= member i's n_out.
 * For T <= 16, when the members share the pattern and code form, none holds the compact form, and
 * (for SBN_OUT_F32) none has k:256 outliers, all members run in one kernel launch (one workgroup
 * per 16 output rows of every member); otherwise the members run one after another.
 * Requires T >= 0, K <= ld_q <= 2^26; T == 0 is a no-op. The outputs must not overlap.
 */
sbn_status sbn_bitlinear_fwd_group(const sbn_packed* const* ws /* host */, int count,
                                   const int8_t* x_q, int64_t ld_q, const float* x_absmax,
                                   int64_t T, void* const* ys /* host */,
                                   const int64_t* ld_ys /* host */, sbn_out_kind out_kind,
                                   void* stream);

/*
 * Grouped quantize-and-multiply: the activation quantization of sbn_quantize_act (after the
 * parameter-free LayerNorm of sbn_layernorm_quantize_act when ln_eps > 0; ln_eps == 0: none),
 * then sbn_bitlinear_fwd_group on the result ("The BitLinear Layer", operations 1, 2, 4 and 5).
 * x_q and x_absmax receive exactly what the quantizer writes; the outputs are exactly those of
 * sbn_bitlinear_fwd_group. For T <= 4 and K <= 12288, under the one-launch conditions of
 * sbn_bitlinear_fwd_group, the whole call is one kernel launch in which every workgroup quantizes
 * the activations it needs itself; otherwise the first member runs as sbn_bitlinear_fwd_bf16
 * (or sbn_bitlinear_fwd_ln_bf16) and the others read its x_q and x_absmax.
 * Requires ld_x >= K, ln_eps >= 0 and finite, and the requirements of sbn_bitlinear_fwd_group.
 */
sbn_status sbn_bitlinear_fwd_group_bf16(const sbn_packed* const* ws /* host */, int count,
                                        const uint16_t* x_bf16, int64_t ld_x, int64_t T,
                                        float ln_eps, int8_t* x_q, int64_t ld_q, float* x_absmax,
                                        void* const* ys /* host */,
                                        const int64_t* ld_ys /* host */, sbn_out_kind out_kind,
                                        void* stream);

/* Bytes of device workspace sbn_bitlinear_fwd_latent_static holds on each device it runs on. */
#define SBN_STATIC_WORKSPACE_BYTES ((size_t)32 << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the pack of sbn_pack_nm_ternary (flags 0) of the
 * latent weights followed by sbn_bitlinear_fwd, with the same results, but with the packed planes,
 * the absmean partial sums and the split-K words in a fixed library-owned device workspace of
 * SBN_STATIC_WORKSPACE_BYTES instead of a handle. The call allocates nothing (no hipMalloc or
 * hipFree, no allocating library routine); it enqueues a fill kernel that clears the workspace
 * regions that must start at zero, the pack kernels and the forward.
 *   Arguments as for sbn_pack_nm_ternary (w_latent, n_out, K, ld_w, n_keep, m_group) and
 *   sbn_bitlinear_fwd (x_q, ld_q, x_absmax, T, y, ld_y, out_kind).
 * A weight whose planes do not fit the workspace gives SBN_ERR_UNSUPPORTED (the 7B-style
 * 4096 x 11008 layers at 2:4 or 8:16 take about 17 MB; the limit is about 88M weights at 2:4).
 * Every call on a device shares that device's workspace, which keeps the last call's contents:
 * calls that overlap on one device (two streams, or two host threads) race and give wrong
 * results; order them. No handle exists, so nothing is exported and no mask flips are counted.
 * T == 0 or n_out == 0 is a no-op.
 */
sbn_status sbn_bitlinear_fwd_latent_static(const float* w_latent, int64_t n_out, int64_t K,
                                           int64_t ld_w, int n_keep, int m_group,
                                           const int8_t* x_q, int64_t ld_q, const float* x_absmax,
                                           int64_t T, void* y, int64_t ld_y,
                                           sbn_out_kind out_kind, void* stream);

/*
 * Data gradient of the layer under the straight-through estimator ("Microsoft BitNet 1.58: The
 * Era of 1-Bit Large Language Models", section "Training with the Straight-Through Estimator":
 * the backward pass treats both quantizers as the identity, so the gradient flows through the
 * ternary weights gamma * C of the last pack).
 *   dy_bf16   [T][ld_dy] bf16 bit patterns (uint16), the gradient of y, read only.
 *   dx        [T][ld_dx] fp32 out: dx[t][k] = fl32( gamma * S ), S = sum_r dy[t][r] * code[r][k]
 *             accumulated in fp32 (every product is exact; the order of the fp32 additions is
 *             unspecified, so |S - exact| <= (n_out - 1) * 2^-24 * sum_r |dy[t][r] * code[r][k]|).
 * The first call after a pack rebuilds the handle's transposed code plane (one extra kernel);
 * later calls reuse it (the kernel still launches and exits at once). Whether a pack has run since
 * is tracked in device memory, so packs and data gradients may be replayed from captured HIP
 * graphs in any mix. n_out == 0 gives dx = 0.
 * Requires T >= 0, n_out <= ld_dy <= 2^25, ld_dx >= K, n_out <= 2^27; T == 0 is a no-op.
 */
sbn_status sbn_bitlinear_bwd_dx(const sbn_packed* w, const uint16_t* dy_bf16, int64_t ld_dy,
                                int64_t T, float* dx, int64_t ld_dx, void* stream);

/*
 * Releases a handle. Where the device supports memory pools (MI355X does), its device memory was
 * allocated stream-ordered and is released stream-ordered on the last stream that used the handle,
 * without blocking the host; otherwise this waits for that stream, then frees. Work on other
 * streams that still uses the handle must be ordered before that stream by the caller.
 * sbn_free(NULL) is a no-op.
 */
void sbn_free(sbn_packed* handle);

/*
 * Canonical export of a handle, for tests and checkpoints (enqueued on `stream`):
 *   codes     [n_out][K] int8 in {-1, 0, +1} (0 where pruned), or NULL to skip
 *   keep_mask [n_out][K] uint8 in {0, 1}, or NULL to skip
 *   gamma     [1] fp32, or NULL to skip (the scale the matmuls use: gamma, or the
 *             variance-corrected gamma_out after a pack with SBN_PACK_VARIANCE_CORRECTION)
 */
sbn_status sbn_packed_export(const sbn_packed* w, int8_t* codes, uint8_t* keep_mask, float* gamma,
                             void* stream);

/*
 * Export of the packed bytes in the reference packed format (RPF): per row, a code bitstream
 * (group g's n kept codes, ascending position, at bits [2n*g, 2n*(g+1)); 2-bit two's complement
 * 00 = 0, 01 = +1, 11 = -1; LSB first) padded to code_row_bytes = ceil(K/m*2n/8), and, when
 * n < m, a mask bitstream (bit i of group g <-> position g*m + i) of mask_row_bytes = ceil(K/8).
 *   code_bytes [n_out][code_row_bytes] uint8, mask_bytes [n_out][mask_row_bytes] uint8
 *   (mask_bytes may be NULL when n == m). Either may be NULL to skip it.
 */
sbn_status sbn_packed_export_rpf(const sbn_packed* w, uint8_t* code_bytes, uint8_t* mask_bytes,
                                 void* stream);

/*
 * Export of the k:256 outliers of the last pack (which must have had SBN_PACK_OUTLIERS(k), else
 * SBN_ERR_INVALID_ARG), enqueued on `stream`:
 *   positions [n_out][K/256][k] uint8, ascending within each group (position in the group)
 *   values    [n_out][K/256][k] uint16, bf16 bit patterns
 * Either may be NULL to skip it.
 */
sbn_status sbn_packed_export_outliers(const sbn_packed* w, uint8_t* positions, uint16_t* values,
                                      void* stream);

/*
 * Export of the compact form written by the last pack (which must have had SBN_PACK_COMPACT, else
 * SBN_ERR_INVALID_ARG), enqueued on `stream`. Per row a bit stream, LSB first, padded to
 * compact_row_bytes = ceil((K/m)(m + n)/8): group g (positions g*m .. g*m+m-1) at bits
 * [g(m+n), (g+1)(m+n)); bit i < m is 1 when position g*m + i holds a nonzero code; bit m + j is 1
 * when the group's j-th nonzero code, counting by ascending position, is -1 (slots past the
 * group's nonzero count are 0).
 *   bytes     [n_out][compact_row_bytes] uint8 out (device).
 */
sbn_status sbn_packed_export_compact(const sbn_packed* w, uint8_t* bytes, void* stream);

/*
 * Export of the last pack's codes in the rank encoding, enqueued on `stream` (any handle, any
 * code form). The pages print n:m metadata sizes of 0.75 bits per element for 2:4 and 0.875 for
 * 8:16 ("From 2:4 to 8:16 sparsity patterns in LLMs for Outliers and Weights with Variance
 * Correction", abstract): R = ceil(log2 C(m, n)) bits per group of m, the width of a fixed-size
 * index of the group's n-of-m choice. Per row a bit stream, LSB first, padded to
 * rank_row_bytes = ceil((K/m)(R + 2n)/8): group g at bits [g(R + 2n), (g+1)(R + 2n)) holds the
 * rank of its keep mask in the combinatorial number system (colex order: the sum, over the i-th
 * kept position c counted from 1 by ascending position, of C(c, i)), then the two's-complement
 * low two bits of its n kept codes by ascending position (0 -> 00, +1 -> 01, -1 -> 11). 2:4 and
 * 8:16 take 1.75 and 1.875 bits per weight. The GEMV does not read this form.
 *   bytes     [n_out][rank_row_bytes] uint8 out (device); every byte is written.
 */
sbn_status sbn_packed_export_rank(const sbn_packed* w, uint8_t* bytes, void* stream);

/*
 * Keep-mask changes of the handle's last pack: the number of positions whose keep bit differs from
 * the pack before it (the first pack of a handle compares against an empty mask, so it counts
 * every kept position). flips / (n_out * K) is the mask flip rate r_t of Sparse-BitNet, Figure 3
 * (b) (the equation's text is not on the page; this is its plainest reading). Always 0 when
 * n == m. Enqueued on `stream`:
 *   flips     [1] uint64 out (device).
 */
sbn_status sbn_packed_mask_flips(const sbn_packed* w, uint64_t* flips, void* stream);

typedef struct {
  int64_t n_out, K;
  int n, m;
  size_t code_row_bytes, mask_row_bytes; /* RPF row sizes */
  size_t rpf_bytes;                      /* n_out * (code_row_bytes + mask_row_bytes) */
  size_t packed_bytes;                   /* bytes the forward kernels stream (kernel layout) */
  size_t device_bytes;                   /* all device memory the handle holds */
  size_t compact_row_bytes;              /* compact export row size, ceil((K/m)(m+n)/8) */
  size_t compact_bytes;                  /* bytes of the compact plane the GEMV streams */
  int compact;                           /* the last pack wrote the compact form */
  int outlier_k;                         /* k of the last pack's k:256 outliers (0: none) */
  size_t rank_row_bytes;                 /* rank export row size, ceil((K/m)(R + 2n)/8) */
  uint32_t splitk_giveups;               /* split-K waits that gave up (0 in a correct run) */
  int single_pass;                       /* the last pack was a single-read re-pack */
} sbn_packed_desc;

/*
 * Describes a handle; `out` is a host pointer. To read splitk_giveups it waits for the handle's
 * last stream. A forward that runs two workgroups per output tile (each half of K; launches with
 * few tiles) passes partial sums through a handshake whose waiting half spins a bounded time; if
 * it ever gives up, that tile is wrong and this counter, kept in the handle's device memory, says
 * how many times it happened.
 */
sbn_status sbn_packed_query(const sbn_packed* w, sbn_packed_desc* out /* host */);

/* The message of the last failed call on this host thread ("" if none). */
const char* sbn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SBN_H */
