/*
 * sdpa.h -- C ABI of libsdpa07: fused scaled-dot-product attention on
 * AMD Instinct MI355X (gfx950).
 *
 * Operation (the plain definition; the pages name it without a formula):
 *   O = softmax(scale * Q K^T + mask) V,  LSE_i = ln sum_{j visible} exp(scale q_i . k_j)
 * "Inside NVIDIA's cuDNN Graph API: Fusion, Autotuning, and Plan Reuse with
 * cuDNN Frontend", section 5 "SDPA (Flash Attention) with causal masking":
 * Q, K, V of logical shape (b, h, s, d), an attention scale, and causal
 * masking as a top-left diagonal band with right bound 0, i.e. query i sees
 * key j iff j <= i (also when s_q != s_kv).
 * cudnn-frontend PR #554 "torch: put torch.sdpa on the cuDNN Python API
 * (CUDNN provider + dense backward)": the forward's optional per-row
 * statistic (aten's logsumexp: fp32, (b, h, s) dense, (T, h) token-major for
 * packed THD); packed THD batches indexed by int32 cu_seqlens prefix sums with
 * max_seqlen bounds and no attention across sequences; the dense backward
 * producing dQ, dK, dV from Q, K, V, O, dO and the statistic; operands whose
 * innermost dimension is dense and whose base is 16-byte aligned.
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is a DEVICE pointer owned by the caller. No call
 *    allocates device memory, and none keeps a pointer after return (the
 *    one fixed array the library holds is described at
 *    sdpa_bwd_ex_noalloc).
 *  - Strides are in ELEMENTS. Dense tensors take 4 strides in logical
 *    (b, h, s, d) order, packed THD tensors 3 strides in (t, h, d) order. The
 *    d stride must be 1; every other stride, and every base pointer, must
 *    keep 16-byte alignment of each row (multiples of 8 elements for
 *    fp16/bf16, 4 for fp32). Any permutation of the outer dimensions works
 *    (BHSD, BSHD, ...).
 *  - One io dtype per call for Q, K, V, O (and dO, dQ, dK, dV); LSE is always
 *    fp32. Accumulation is fp32.
 *  - Head dims d in {64, 128}.
 *  - `stream` is a hipStream_t (NULL = the null stream). Every call only
 *    enqueues kernels on it and returns; nothing is synchronised and device
 *    memory is never read by the host. Calls are thread-safe, except that
 *    overlapping sdpa_bwd_ex_noalloc calls on one device share its fixed
 *    workspace.
 *  - A row with no visible key (s_kv = 0, or a packed sequence with no keys)
 *    gets O = 0 and LSE = -inf. Sizes of zero return SDPA_OK without
 *    launching.
 *  - Errors: functions never throw. On a non-OK status, sdpa_last_error()
 *    returns a message for the calling thread.
 *      SDPA_ERR_INVALID_ARG  null required pointer, negative size, non-finite
 *                            scale, bad workspace, int32 index overflow
 *      SDPA_ERR_UNSUPPORTED  dtype, head dim, d stride != 1, misaligned base
 *                            pointer or stride
 *      SDPA_ERR_LAUNCH       the HIP runtime rejected a launch
 */
#ifndef SDPA07_SDPA_H
#define SDPA07_SDPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SDPA_OK = 0,
  SDPA_ERR_INVALID_ARG = 1,
  SDPA_ERR_UNSUPPORTED = 2,
  SDPA_ERR_LAUNCH = 3
} sdpa_status;

/* SDPA_FP8_E4M3 (OCP FP8 E4M3, one byte per element) is accepted only by
 * the sdpa_fwd_fp8* entry points, as their input type. */
typedef enum { SDPA_FP32 = 0, SDPA_FP16 = 1, SDPA_BF16 = 2, SDPA_FP8_E4M3 = 3 } sdpa_dtype;

/*
 * Dense forward.
 *   q: (b, h, s_q, d)   k, v: (b, h, s_kv, d)   o: (b, h, s_q, d), written
 *   lse: fp32 (b, h, s_q) contiguous, written; may be NULL (not produced)
 *   scale: multiplies Q K^T (pass 1/sqrt(d) for the usual scaling)
 *   causal: 0 or 1 (top-left)
 * Cited: the cuDNN Graph API article, section 5 (operation, scale, causal);
 * cudnn-frontend PR #554 (statistic layout (B, H, S) fp32).
 */
sdpa_status sdpa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     sdpa_dtype dtype, int b, int h, int s_q, int s_kv, int d,
                     const int64_t q_stride[4], const int64_t k_stride[4],
                     const int64_t v_stride[4], const int64_t o_stride[4], float scale,
                     int causal, void* stream);

/*
 * Packed THD (varlen) forward.
 *   q, o: (total_q, h, d); k, v: (total_kv, h, d); strides in (t, h, d) order.
 *   cu_seqlens_q, cu_seqlens_kv: DEVICE int32 [num_seqs + 1], non-decreasing,
 *     cu[0] = 0, cu[num_seqs] <= total. Sequence n owns tokens
 *     [cu[n], cu[n+1]); positions (and the causal test) are local to it.
 *   max_seqlen_q, max_seqlen_kv: upper bounds on the query and key lengths
 *     (checked > 0 and <= the totals; the kernels take the lengths
 *     themselves from cu_seqlens).
 *   lse: fp32 (total_q, h) token-major contiguous; may be NULL.
 * The grid holds total_q / 256 + num_seqs units per head (pairs of 128-row
 * query tiles; total_q / 128 + num_seqs single tiles for fp32 and e4m3),
 * a bound on the live units of any batch that meets the contract below;
 * each workgroup finds its unit from cu_seqlens on the device, the units
 * of all sequences in decreasing order of work.
 * The cu_seqlens contents are a caller contract (the host never reads them);
 * the kernels clamp every row index to [0, total) so rows at or beyond
 * total_q / total_kv (e.g. an allocation's capacity tail) are never read or
 * written, and query rows beyond a sequence's length are never written.
 * Offsets that break the contract (decreasing, or summing past the totals)
 * are still never followed outside [0, total), but rows of such a batch may
 * be left unwritten.
 * Cited: cudnn-frontend PR #554 (THD packing with cu_seqlens and max_seqlen,
 * (T, H, 1) token-major statistic); its merge log, the FP8 d512 forward entry
 * (keys past the packed total must not feed P.V; dead rows get -inf).
 */
sdpa_status sdpa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                            int num_seqs, int total_q, int total_kv, int max_seqlen_q,
                            int max_seqlen_kv, sdpa_dtype dtype, int h, int d,
                            const int64_t q_stride[3], const int64_t k_stride[3],
                            const int64_t v_stride[3], const int64_t o_stride[3], float scale,
                            int causal, void* stream);

/*
 * Dense forward with grouped-query heads and the band options.
 *   As sdpa_fwd, with:
 *   h, h_kv: query heads and key/value heads; h must be a positive multiple
 *     of h_kv, and query head i reads K/V head i / (h / h_kv) (h_kv == h is
 *     plain multi-head attention, h_kv == 1 multi-query); k, v are
 *     (b, h_kv, s_kv, d).
 *   causal: 0 or 1: keys right of the aligned diagonal are hidden.
 *   bottom_right: 0 aligns the diagonal top-left (query i with key i), 1
 *     bottom-right (query i with key i + s_kv - s_q); 1 needs causal or a
 *     window (SDPA_ERR_INVALID_ARG otherwise).
 *   window_left: -1 for none, else W >= 0: keys more than W left of the
 *     aligned diagonal are hidden (query i keeps keys p - W .. p, and with
 *     causal = 0 every key from p - W on, where p is its diagonal key).
 *   Rows left with no visible key get O = 0 and LSE = -inf.
 * Cited: cudnn-frontend PR #554, the sdpa API (is_causal, causal_bottom_right,
 * window_left; bottom-right without an active band is rejected) and the
 * provider's GQA support; the cuDNN Graph API article, section 5 (the
 * causal mask as a diagonal band with right bound 0).
 */
sdpa_status sdpa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                        sdpa_dtype dtype, int b, int h, int h_kv, int s_q, int s_kv, int d,
                        const int64_t q_stride[4], const int64_t k_stride[4],
                        const int64_t v_stride[4], const int64_t o_stride[4], float scale,
                        int causal, int bottom_right, int window_left, void* stream);

/*
 * Packed THD forward with grouped-query heads and the band options (as
 * sdpa_fwd_varlen and sdpa_fwd_ex): k, v are (total_kv, h_kv, d); the
 * bottom-right alignment uses each sequence's own lengths.
 */
sdpa_status sdpa_fwd_varlen_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                               int num_seqs, int total_q, int total_kv, int max_seqlen_q,
                               int max_seqlen_kv, sdpa_dtype dtype, int h, int h_kv, int d,
                               const int64_t q_stride[3], const int64_t k_stride[3],
                               const int64_t v_stride[3], const int64_t o_stride[3], float scale,
                               int causal, int bottom_right, int window_left, void* stream);

/*
 * FP8 forward, dense: Q, K, V hold e4m3 codes (OCP FP8 E4M3, strides in
 * bytes-as-elements, rows 16-byte aligned), O is written in o_dtype
 * (SDPA_BF16 or SDPA_FP16).
 *   descale_q, descale_k, descale_v, scale_o: DEVICE pointers to one fp32
 *     each, read by the kernel (NULL means 1): the attention runs on
 *     descale_q * Q, descale_k * K, descale_v * V and stores scale_o * O.
 *   amax_o: DEVICE pointer to one fp32 or NULL: set to max |stored O| over
 *     every row, before the cast to o_dtype (the library clears it first).
 *   lse: as in sdpa_fwd, the statistic of the real scores
 *     scale * descale_q * descale_k * Q K^T.
 *   Grouped-query heads and the mask options as in sdpa_fwd_ex.
 * P (the softmax numerator, at most 2^8 of the row's running offset) is
 * rounded to e4m3 before the P.V product and l sums the rounded values, so
 * O differs from the exact result by the rounding of P (relative step 2^-3
 * per element); the scores are exact products accumulated in fp32.
 * Cited: cudnn-frontend PR #554, its merge log's per-tensor FP8 d512 forward
 * entry (descales read on the device, descale_q * descale_k folded into the
 * log2 softmax scale, descale_v * scale_o into the output factor, Amax_O of
 * the fp32 output before the cast) and its FP8 forward casting P before the
 * second product.
 */
sdpa_status sdpa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                         const float* descale_q, const float* descale_k, const float* descale_v,
                         const float* scale_o, float* amax_o, sdpa_dtype o_dtype, int b, int h,
                         int h_kv, int s_q, int s_kv, int d, const int64_t q_stride[4],
                         const int64_t k_stride[4], const int64_t v_stride[4],
                         const int64_t o_stride[4], float scale, int causal, int bottom_right,
                         int window_left, void* stream);

/*
 * FP8 forward, packed THD (as sdpa_fwd_varlen_ex, with the fp8 arguments of
 * sdpa_fwd_fp8): q (total_q, h, d), k, v (total_kv, h_kv, d) e4m3 codes.
 */
sdpa_status sdpa_fwd_fp8_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                const float* descale_q, const float* descale_k,
                                const float* descale_v, const float* scale_o, float* amax_o,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                int num_seqs, int total_q, int total_kv, int max_seqlen_q,
                                int max_seqlen_kv, sdpa_dtype o_dtype, int h, int h_kv, int d,
                                const int64_t q_stride[3], const int64_t k_stride[3],
                                const int64_t v_stride[3], const int64_t o_stride[3],
                                float scale, int causal, int bottom_right, int window_left,
                                void* stream);

/*
 * Bytes of device workspace the backward needs for these sizes: two fp32
 * values per query row (rowsum(dO * O) and the statistic in base 2), rounded
 * up to 256 bytes. The caller allocates it (256-byte aligned) and passes it to
 * sdpa_bwd*, so the library itself never allocates. For the packed backward
 * pass b = 1, s_q = total_q. Returns 256 for empty problems; never fails.
 * Cited: the cuDNN Graph API article, section 5: the caller sizes and
 * allocates the device workspace of the built attention operation (its
 * workspace_for / get_workspace_size step) and hands it to every execute
 * call; cudnn-frontend PR #554's merge log (the SM80 backward entry) names
 * the dO.O row dot product that this workspace holds.
 */
size_t sdpa_bwd_workspace_size(int b, int h, int s_q, int d, sdpa_dtype dtype);

/*
 * Dense backward (fp16/bf16).
 *   q, k, v, o, dout as in sdpa_fwd (o is the forward's output, dout = dL/dO);
 *   lse: fp32 (b, h, s_q) contiguous, the forward's statistic (required);
 *   dq, dk, dv: written, same logical shapes as q, k, v, with their own
 *     strides (e.g. the inputs' permutation);
 *   workspace: device buffer of at least sdpa_bwd_workspace_size() bytes,
 *     256-byte aligned; its contents on entry are ignored.
 * Deterministic: no atomics; repeated calls give bit-identical gradients.
 * Two kernels on `stream`: a dQ pass, which also forms rowsum(dO * O) and
 * the base-2 statistic into the workspace, then a dK/dV pass that reads them.
 * Cited: cudnn-frontend PR #554 (dense backward, gradients in the inputs'
 * layouts, deterministic flag honoured); its merge log, the SM80 backward
 * TemplateParams entry (the chain starts with the dO.O row dot product).
 */
sdpa_status sdpa_bwd(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes, sdpa_dtype dtype, int b, int h,
                     int s_q, int s_kv, int d, const int64_t q_stride[4],
                     const int64_t k_stride[4], const int64_t v_stride[4],
                     const int64_t o_stride[4], const int64_t do_stride[4],
                     const int64_t dq_stride[4], const int64_t dk_stride[4],
                     const int64_t dv_stride[4], float scale, int causal, void* stream);

/*
 * Dense backward with grouped-query heads and the band options; the mask
 * arguments are those of sdpa_fwd_ex and must match the forward call that
 * produced o and lse.
 *   k, v, dk, dv are (b, h_kv, s_kv, d); dK and dV of K/V head j sum the
 *   contributions of query heads j * (h / h_kv) .. (j + 1) * (h / h_kv) - 1.
 *   Keys no query sees get dK = dV = 0; queries that see no key get dQ = 0.
 * Row strides must keep a 128-row tile within 2 GiB (SDPA_ERR_UNSUPPORTED).
 * Cited: cudnn-frontend PR #554 (the sdpa backward takes the forward's mask
 * options; GQA support in the provider); the cuDNN Graph API article,
 * section 5 (the band mask).
 */
sdpa_status sdpa_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, sdpa_dtype dtype, int b, int h,
                        int h_kv, int s_q, int s_kv, int d, const int64_t q_stride[4],
                        const int64_t k_stride[4], const int64_t v_stride[4],
                        const int64_t o_stride[4], const int64_t do_stride[4],
                        const int64_t dq_stride[4], const int64_t dk_stride[4],
                        const int64_t dv_stride[4], float scale, int causal, int bottom_right,
                        int window_left, void* stream);

/*
 * sdpa_bwd_ex without a workspace argument, for callers that cannot allocate
 * device memory: code under stream capture, tight serving loops, harnesses
 * that forbid allocation. Arguments, results and errors are those of
 * sdpa_bwd_ex; the caller still provides every input and output.
 *   The workspace is a fixed array in the library's device code,
 *   SDPA_BWD_FIXED_WORKSPACE_BYTES (16 MiB) on each device the library runs
 *   on, held until the process ends. It serves b * h * s_q up to
 *   SDPA_BWD_FIXED_WORKSPACE_ROWS (2^21) query rows; more is rejected with
 *   SDPA_ERR_UNSUPPORTED before anything is launched.
 *   Allocates nothing: no hipMalloc / hipFree. The first call on a device
 *   (the current device, which `stream` must belong to) looks up the array's
 *   device address once; failure there is SDPA_ERR_LAUNCH.
 *   Every call on one device uses that device's one array: calls that
 *   overlap on a device (other streams, other threads) race and must be
 *   serialised by the caller. Each call writes every workspace value it
 *   reads, so what an earlier call left there does not matter.
 */
#define SDPA_BWD_FIXED_WORKSPACE_BYTES (16u << 20)
#define SDPA_BWD_FIXED_WORKSPACE_ROWS (1 << 21)
sdpa_status sdpa_bwd_ex_noalloc(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                sdpa_dtype dtype, int b, int h, int h_kv, int s_q, int s_kv,
                                int d, const int64_t q_stride[4], const int64_t k_stride[4],
                                const int64_t v_stride[4], const int64_t o_stride[4],
                                const int64_t do_stride[4], const int64_t dq_stride[4],
                                const int64_t dk_stride[4], const int64_t dv_stride[4],
                                float scale, int causal, int bottom_right, int window_left,
                                void* stream);

/*
 * Packed THD backward (fp16/bf16), with grouped-query heads and the band
 * options as sdpa_bwd_ex.
 *   q, o, dout, dq: (total_q, h, d); k, v, dk, dv: (total_kv, h_kv, d); each
 *     with its own (token, head) strides and d stride 1;
 *   lse: fp32 (total_q, h) token-major, as written by sdpa_fwd_varlen(_ex);
 *   cu_seqlens_q / cu_seqlens_kv, num_seqs, total_*, max_seqlen_*: as in
 *     sdpa_fwd_varlen (device int32 arrays of num_seqs + 1 entries; the
 *     dK/dV and dQ grids hold total / 128 + num_seqs tiles per head and
 *     their workgroups find their tiles from cu_seqlens);
 *   workspace: sdpa_bwd_workspace_size(1, h, total_q, d, dtype) bytes.
 * Rows at or past total_q / total_kv are never read or written; rows of
 * sequences with no keys get dQ = 0, rows of sequences with no queries
 * get dK = dV = 0. Deterministic (no atomics).
 * Cited: cudnn-frontend PR #554 (THD packing with cu_seqlens and max_seqlen,
 * the (T, H, 1) token-major statistic shared by forward and backward).
 */
sdpa_status sdpa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                            int num_seqs, int total_q, int total_kv, int max_seqlen_q,
                            int max_seqlen_kv, void* workspace, size_t workspace_bytes,
                            sdpa_dtype dtype, int h, int h_kv, int d, const int64_t q_stride[3],
                            const int64_t k_stride[3], const int64_t v_stride[3],
                            const int64_t o_stride[3], const int64_t do_stride[3],
                            const int64_t dq_stride[3], const int64_t dk_stride[3],
                            const int64_t dv_stride[3], float scale, int causal,
                            int bottom_right, int window_left, void* stream);

/*
 * Message for the calling thread's last non-OK status ("" after a call that
 * returned SDPA_OK). The string is owned by the library, stays valid until
 * the calling thread's next sdpa_* call, and is never NULL.
 * Cited: TransformerEngine PR #2964 "Refactor nvte_get_fused_attn_backend
 * with cudnn-frontend calls": the support probe reports the backend's own
 * error message as a string (empty when supported) instead of a bare
 * "no backend" answer.
 */
const char* sdpa_last_error(void);

/* Library version string. */
const char* sdpa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDPA07_SDPA_H */
