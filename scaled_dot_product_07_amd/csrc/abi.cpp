// C ABI of libsdpa07 (declared in include/sdpa.h): argument validation and
// kernel dispatch. Validation never touches device memory and never
// synchronises, so every status path can be exercised without a GPU.
//
// The checks follow what the pages require of operands: dense innermost
// dimension and 16-byte aligned base (cudnn-frontend PR #554, the dense
// operand normalisation commit: a strided last dim or a misaligned base must
// fail loudly instead of reading wrong elements); THD needs cu_seqlens and
// positive max_seqlen bounds (same pull request, the varlen validation); a
// status plus a message instead of an exception (TransformerEngine PR #2964,
// backend probe returning an error string).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "sdpa.h"
#include "sdpa_internal.h"

namespace {

thread_local std::string g_last_error;

sdpa_status fail(sdpa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

sdpa_status ok() {
  g_last_error.clear();
  return SDPA_OK;
}

int elem_size(sdpa_dtype dt) { return dt == SDPA_FP32 ? 4 : dt == SDPA_FP8_E4M3 ? 1 : 2; }

bool valid_dtype(sdpa_dtype dt) { return dt == SDPA_FP32 || dt == SDPA_FP16 || dt == SDPA_BF16; }

// Strides of one tensor with `nd` dims (outer dims first, d last) and the
// dim sizes. A dimension of size 1 may carry any stride.
sdpa_status check_tensor(const char* name, const void* ptr, const int64_t* st, const int* sizes,
                         int nd, sdpa_dtype dt, bool needed) {
  if (!st) return fail(SDPA_ERR_INVALID_ARG, "%s: stride array is NULL", name);
  if (!needed) return SDPA_OK;
  if (!ptr) return fail(SDPA_ERR_INVALID_ARG, "%s: NULL pointer", name);
  if (st[nd - 1] != 1)
    return fail(SDPA_ERR_UNSUPPORTED, "%s: innermost (d) stride is %lld, must be 1", name,
                (long long)st[nd - 1]);
  const int es = elem_size(dt);
  if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
    return fail(SDPA_ERR_UNSUPPORTED, "%s: base pointer is not 16-byte aligned", name);
  for (int i = 0; i < nd - 1; ++i) {
    if (sizes[i] <= 1) continue;
    if (st[i] < 0)
      return fail(SDPA_ERR_UNSUPPORTED, "%s: negative stride %lld in dim %d", name,
                  (long long)st[i], i);
    if ((st[i] * es) % 16 != 0)
      return fail(SDPA_ERR_UNSUPPORTED,
                  "%s: stride %lld of dim %d breaks 16-byte row alignment", name,
                  (long long)st[i], i);
  }
  return SDPA_OK;
}

// Key rows are streamed in tiles addressed with 32-bit byte offsets from the
// tile's first row: a tile of kTileRows rows must span less than 2 GiB.
sdpa_status check_tile_span(const char* name, int64_t row_stride, sdpa_dtype dt) {
  constexpr int64_t kTileRows = 128;
  const int64_t span = (row_stride < 0 ? -row_stride : row_stride) * elem_size(dt) * kTileRows;
  if (span >= 0x7fffffffLL)
    return fail(SDPA_ERR_UNSUPPORTED, "%s: row stride %lld too large for 32-bit tile offsets", name,
                (long long)row_stride);
  return SDPA_OK;
}

sdpa07::Dt to_dt(sdpa_dtype dt) {
  return dt == SDPA_FP32 ? sdpa07::Dt::F32 : dt == SDPA_FP16 ? sdpa07::Dt::F16 : sdpa07::Dt::BF16;
}

float scale_log2(float scale) {
  // |scale| * log2(e), kept strictly positive so that -inf masks stay -inf
  // after the scaling even for scale = 0 (then every visible key weighs 1).
  const float c = std::fabs(scale) * 1.4426950408889634f;
  return c > 1e-30f ? c : 1e-30f;
}

bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("SDPA07_LOG");
    return e && e[0] == '1';
  }();
  return on;
}

sdpa_status launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(SDPA_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

// Mask options (cudnn-frontend PR #554's sdpa API: is_causal,
// causal_bottom_right, window_left; bottom-right alignment needs a band).
sdpa_status check_mask(int causal, int bottom_right, int window_left) {
  if (causal != 0 && causal != 1) return fail(SDPA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (bottom_right != 0 && bottom_right != 1)
    return fail(SDPA_ERR_INVALID_ARG, "bottom_right must be 0 or 1");
  if (window_left < -1)
    return fail(SDPA_ERR_INVALID_ARG, "window_left %d (expected >= 0, or -1 for none)",
                window_left);
  if (bottom_right && !causal && window_left < 0)
    return fail(SDPA_ERR_INVALID_ARG, "bottom_right needs causal or a window_left >= 0");
  return SDPA_OK;
}

// Query heads h read K/V head i / (h / h_kv): h a positive multiple of h_kv.
sdpa_status check_heads(int h, int h_kv) {
  if (h_kv < 0) return fail(SDPA_ERR_INVALID_ARG, "negative h_kv %d", h_kv);
  if (h > 0 && (h_kv == 0 || h % h_kv != 0))
    return fail(SDPA_ERR_INVALID_ARG, "h_q %d is not a multiple of h_kv %d", h, h_kv);
  return SDPA_OK;
}

// Workspace checks shared by both backward entry points.
sdpa_status check_workspace(const void* workspace, size_t workspace_bytes, long long rows) {
  if (!workspace) return fail(SDPA_ERR_INVALID_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(SDPA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  const size_t need = sdpa07::bwd_workspace_bytes(rows);
  if (workspace_bytes < need)
    return fail(SDPA_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu needed",
                workspace_bytes, need);
  return SDPA_OK;
}

// Arguments only the fp8 entry points take.
sdpa_status check_fp8_extras(sdpa_dtype o_dtype, const float* descale_q, const float* descale_k,
                             const float* descale_v, const float* scale_o, const float* amax_o) {
  if (o_dtype != SDPA_BF16 && o_dtype != SDPA_FP16)
    return fail(SDPA_ERR_UNSUPPORTED, "fp8 forward writes bf16 or fp16 output, not dtype %d",
                (int)o_dtype);
  const float* ptrs[5] = {descale_q, descale_k, descale_v, scale_o, amax_o};
  const char* names[5] = {"descale_q", "descale_k", "descale_v", "scale_o", "amax_o"};
  for (int i = 0; i < 5; ++i)
    if (reinterpret_cast<uintptr_t>(ptrs[i]) % 4 != 0)
      return fail(SDPA_ERR_UNSUPPORTED, "%s: pointer is not 4-byte aligned", names[i]);
  return SDPA_OK;
}

}  // namespace

extern "C" {

const char* sdpa_last_error(void) { return g_last_error.c_str(); }

const char* sdpa_version(void) { return "sdpa07 0.1.0 gfx950"; }

sdpa_status sdpa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                        sdpa_dtype dtype, int b, int h, int h_kv, int s_q, int s_kv, int d,
                        const int64_t q_stride[4], const int64_t k_stride[4],
                        const int64_t v_stride[4], const int64_t o_stride[4], float scale,
                        int causal, int bottom_right, int window_left, void* stream) {
  if (!valid_dtype(dtype)) return fail(SDPA_ERR_UNSUPPORTED, "unsupported dtype %d", (int)dtype);
  if (b < 0 || h < 0 || s_q < 0 || s_kv < 0 || d < 0)
    return fail(SDPA_ERR_INVALID_ARG, "negative size (b=%d h=%d s_q=%d s_kv=%d d=%d)", b, h, s_q,
                s_kv, d);
  if (d != 64 && d != 128) return fail(SDPA_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d);
  if (!std::isfinite(scale)) return fail(SDPA_ERR_INVALID_ARG, "scale is not finite");
  sdpa_status st;
  if ((st = check_mask(causal, bottom_right, window_left)) != SDPA_OK) return st;
  if ((st = check_heads(h, h_kv)) != SDPA_OK) return st;
  const bool work = b > 0 && h > 0 && s_q > 0;
  const int qs[4] = {b, h, s_q, d}, ks[4] = {b, h_kv, s_kv, d};
  if ((st = check_tensor("q", q, q_stride, qs, 4, dtype, work)) != SDPA_OK) return st;
  if ((st = check_tensor("o", o, o_stride, qs, 4, dtype, work)) != SDPA_OK) return st;
  if ((st = check_tensor("k", k, k_stride, ks, 4, dtype, work && s_kv > 0)) != SDPA_OK) return st;
  if ((st = check_tensor("v", v, v_stride, ks, 4, dtype, work && s_kv > 0)) != SDPA_OK) return st;
  if (lse && reinterpret_cast<uintptr_t>(lse) % 4 != 0)
    return fail(SDPA_ERR_UNSUPPORTED, "lse: pointer is not 4-byte aligned");
  if ((st = check_tile_span("k", k_stride[2], dtype)) != SDPA_OK) return st;
  if ((st = check_tile_span("v", v_stride[2], dtype)) != SDPA_OK) return st;
  const long long n_qtiles = (s_q + sdpa07::kFwdBlockM - 1) / sdpa07::kFwdBlockM;
  if ((long long)b * h * n_qtiles > 0x7fffffffLL)
    return fail(SDPA_ERR_INVALID_ARG, "grid of %lld workgroups exceeds int32",
                (long long)b * h * n_qtiles);
  if (!work) return ok();

  sdpa07::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.q_sb = q_stride[0]; p.q_sh = q_stride[1]; p.q_ss = q_stride[2];
  p.k_sb = k_stride[0]; p.k_sh = k_stride[1]; p.k_ss = k_stride[2];
  p.v_sb = v_stride[0]; p.v_sh = v_stride[1]; p.v_ss = v_stride[2];
  p.o_sb = o_stride[0]; p.o_sh = o_stride[1]; p.o_ss = o_stride[2];
  p.b = b; p.h = h; p.h_kv = h_kv; p.s_q = s_q; p.s_kv = s_kv;
  p.bottom_right = bottom_right; p.window_left = window_left;
  // Options that describe the same band take the same schedule: a left
  // window at least as wide as the longer side cuts no key (every row's
  // lower bound i + shift - window is below key 0), and with equal sides, or
  // with neither bound left, the alignment changes nothing.
  if (p.window_left >= (s_q > s_kv ? s_q : s_kv)) p.window_left = -1;
  if (p.window_left < 0 && (!causal || s_q == s_kv)) p.bottom_right = 0;
  p.n_qtiles = (int)n_qtiles;
  p.scale_log2 = scale_log2(scale);
  p.negate_q = scale < 0.f;
  if (log_enabled())
    fprintf(stderr,
            "[sdpa07] fwd dtype=%d b=%d h=%d h_kv=%d s_q=%d s_kv=%d d=%d causal=%d br=%d "
            "window=%d\n",
            (int)dtype, b, h, h_kv, s_q, s_kv, d, causal, bottom_right, window_left);
  return launch_status(sdpa07::launch_fwd(p, to_dt(dtype), d, causal != 0, false,
                                          (hipStream_t)stream),
                       "sdpa_fwd");
}

sdpa_status sdpa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     sdpa_dtype dtype, int b, int h, int s_q, int s_kv, int d,
                     const int64_t q_stride[4], const int64_t k_stride[4],
                     const int64_t v_stride[4], const int64_t o_stride[4], float scale,
                     int causal, void* stream) {
  return sdpa_fwd_ex(q, k, v, o, lse, dtype, b, h, h, s_q, s_kv, d, q_stride, k_stride, v_stride,
                     o_stride, scale, causal, 0, -1, stream);
}

sdpa_status sdpa_fwd_varlen_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                               int num_seqs, int total_q, int total_kv, int max_seqlen_q,
                               int max_seqlen_kv, sdpa_dtype dtype, int h, int h_kv, int d,
                               const int64_t q_stride[3], const int64_t k_stride[3],
                               const int64_t v_stride[3], const int64_t o_stride[3], float scale,
                               int causal, int bottom_right, int window_left, void* stream) {
  if (!valid_dtype(dtype)) return fail(SDPA_ERR_UNSUPPORTED, "unsupported dtype %d", (int)dtype);
  if (num_seqs < 0 || total_q < 0 || total_kv < 0 || h < 0 || d < 0 || max_seqlen_q < 0 ||
      max_seqlen_kv < 0)
    return fail(SDPA_ERR_INVALID_ARG, "negative size");
  if (d != 64 && d != 128) return fail(SDPA_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d);
  if (!std::isfinite(scale)) return fail(SDPA_ERR_INVALID_ARG, "scale is not finite");
  {
    sdpa_status st0;
    if ((st0 = check_mask(causal, bottom_right, window_left)) != SDPA_OK) return st0;
    if ((st0 = check_heads(h, h_kv)) != SDPA_OK) return st0;
  }
  const bool work = num_seqs > 0 && h > 0 && total_q > 0;
  if (work && (!cu_seqlens_q || !cu_seqlens_kv))
    return fail(SDPA_ERR_INVALID_ARG, "packed path needs cu_seqlens_q and cu_seqlens_kv");
  if (work && (max_seqlen_q <= 0 || max_seqlen_kv <= 0))
    return fail(SDPA_ERR_INVALID_ARG, "packed path needs max_seqlen_q > 0 and max_seqlen_kv > 0");
  if (work && max_seqlen_q > total_q)
    return fail(SDPA_ERR_INVALID_ARG, "max_seqlen_q %d exceeds total_q %d", max_seqlen_q,
                total_q);
  const int qs[3] = {total_q, h, d}, ks[3] = {total_kv, h_kv, d};
  sdpa_status st;
  if ((st = check_tensor("q", q, q_stride, qs, 3, dtype, work)) != SDPA_OK) return st;
  if ((st = check_tensor("o", o, o_stride, qs, 3, dtype, work)) != SDPA_OK) return st;
  if ((st = check_tensor("k", k, k_stride, ks, 3, dtype, work && total_kv > 0)) != SDPA_OK)
    return st;
  if ((st = check_tensor("v", v, v_stride, ks, 3, dtype, work && total_kv > 0)) != SDPA_OK)
    return st;
  if (lse && reinterpret_cast<uintptr_t>(lse) % 4 != 0)
    return fail(SDPA_ERR_UNSUPPORTED, "lse: pointer is not 4-byte aligned");
  if ((st = check_tile_span("k", k_stride[0], dtype)) != SDPA_OK) return st;
  if ((st = check_tile_span("v", v_stride[0], dtype)) != SDPA_OK) return st;
  const long long n_qtiles = (max_seqlen_q + sdpa07::kFwdBlockM - 1) / sdpa07::kFwdBlockM;
  // one workgroup per live query tile (or pair of tiles) per head, bounded
  // from the totals (the kernels find their units from cu_seqlens)
  if (sdpa07::packed_units_per_head(total_q, num_seqs, sdpa07::kFwdBlockM) * h > 0x7fffffffLL)
    return fail(SDPA_ERR_INVALID_ARG, "grid exceeds int32");
  if (!work) return ok();

  sdpa07::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.q_ss = q_stride[0]; p.q_sh = q_stride[1];
  p.k_ss = k_stride[0]; p.k_sh = k_stride[1];
  p.v_ss = v_stride[0]; p.v_sh = v_stride[1];
  p.o_ss = o_stride[0]; p.o_sh = o_stride[1];
  p.b = num_seqs; p.h = h; p.h_kv = h_kv;
  p.bottom_right = bottom_right; p.window_left = window_left;
  p.n_qtiles = (int)n_qtiles;
  p.scale_log2 = scale_log2(scale);
  p.negate_q = scale < 0.f;
  p.cu_q = cu_seqlens_q; p.cu_kv = cu_seqlens_kv;
  p.total_q = total_q; p.total_kv = total_kv;
  if (log_enabled())
    fprintf(stderr, "[sdpa07] fwd_varlen dtype=%d n=%d h=%d T_q=%d T_kv=%d max_q=%d d=%d causal=%d\n",
            (int)dtype, num_seqs, h, total_q, total_kv, max_seqlen_q, d, causal);
  return launch_status(sdpa07::launch_fwd(p, to_dt(dtype), d, causal != 0, true,
                                          (hipStream_t)stream),
                       "sdpa_fwd_varlen");
}

sdpa_status sdpa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                            int num_seqs, int total_q, int total_kv, int max_seqlen_q,
                            int max_seqlen_kv, sdpa_dtype dtype, int h, int d,
                            const int64_t q_stride[3], const int64_t k_stride[3],
                            const int64_t v_stride[3], const int64_t o_stride[3], float scale,
                            int causal, void* stream) {
  return sdpa_fwd_varlen_ex(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_kv, num_seqs, total_q,
                            total_kv, max_seqlen_q, max_seqlen_kv, dtype, h, h, d, q_stride,
                            k_stride, v_stride, o_stride, scale, causal, 0, -1, stream);
}

size_t sdpa_bwd_workspace_size(int b, int h, int s_q, int d, sdpa_dtype dtype) {
  (void)d;
  (void)dtype;
  if (b <= 0 || h <= 0 || s_q <= 0) return 256;
  return sdpa07::bwd_workspace_bytes((long long)b * h * s_q);
}

static_assert(SDPA_BWD_FIXED_WORKSPACE_BYTES == sdpa07::kBwdFixedWorkspaceBytes &&
                  SDPA_BWD_FIXED_WORKSPACE_ROWS == sdpa07::kBwdFixedWorkspaceRows,
              "the header states the fixed workspace's size");

namespace {

// The dense backward of sdpa_bwd_ex and sdpa_bwd_ex_noalloc. With `fixed`,
// `workspace` is ignored and the library's own per-device array takes its
// place (looked up after every check has passed, so that a rejected call
// touches no device state).
sdpa_status bwd_dense(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, bool fixed, sdpa_dtype dtype,
                      int b, int h, int h_kv, int s_q, int s_kv, int d, const int64_t q_stride[4],
                      const int64_t k_stride[4], const int64_t v_stride[4],
                      const int64_t o_stride[4], const int64_t do_stride[4],
                      const int64_t dq_stride[4], const int64_t dk_stride[4],
                      const int64_t dv_stride[4], float scale, int causal, int bottom_right,
                      int window_left, void* stream, const char* what) {
  if (!valid_dtype(dtype)) return fail(SDPA_ERR_UNSUPPORTED, "unsupported dtype %d", (int)dtype);
  if (dtype == SDPA_FP32)
    return fail(SDPA_ERR_UNSUPPORTED, "backward supports fp16 and bf16 io only");
  if (b < 0 || h < 0 || s_q < 0 || s_kv < 0 || d < 0)
    return fail(SDPA_ERR_INVALID_ARG, "negative size");
  if (d != 64 && d != 128) return fail(SDPA_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d);
  if (!std::isfinite(scale)) return fail(SDPA_ERR_INVALID_ARG, "scale is not finite");
  sdpa_status st;
  if ((st = check_mask(causal, bottom_right, window_left)) != SDPA_OK) return st;
  if ((st = check_heads(h, h_kv)) != SDPA_OK) return st;
  const bool work = b > 0 && h > 0 && (s_q > 0 || s_kv > 0);
  const bool qwork = work && s_q > 0, kwork = work && s_kv > 0;
  const int qs[4] = {b, h, s_q, d}, ks[4] = {b, h_kv, s_kv, d};
  if ((st = check_tensor("q", q, q_stride, qs, 4, dtype, qwork && kwork)) != SDPA_OK) return st;
  if ((st = check_tensor("o", o, o_stride, qs, 4, dtype, qwork && kwork)) != SDPA_OK) return st;
  if ((st = check_tensor("dout", dout, do_stride, qs, 4, dtype, qwork && kwork)) != SDPA_OK)
    return st;
  if ((st = check_tensor("dq", dq, dq_stride, qs, 4, dtype, qwork)) != SDPA_OK) return st;
  if ((st = check_tensor("k", k, k_stride, ks, 4, dtype, qwork && kwork)) != SDPA_OK) return st;
  if ((st = check_tensor("v", v, v_stride, ks, 4, dtype, qwork && kwork)) != SDPA_OK) return st;
  if ((st = check_tensor("dk", dk, dk_stride, ks, 4, dtype, kwork)) != SDPA_OK) return st;
  if ((st = check_tensor("dv", dv, dv_stride, ks, 4, dtype, kwork)) != SDPA_OK) return st;
  if ((st = check_tile_span("q", q_stride[2], dtype)) != SDPA_OK) return st;
  if ((st = check_tile_span("dout", do_stride[2], dtype)) != SDPA_OK) return st;
  if ((st = check_tile_span("k", k_stride[2], dtype)) != SDPA_OK) return st;
  if ((st = check_tile_span("v", v_stride[2], dtype)) != SDPA_OK) return st;
  if (qwork && kwork && !lse)
    return fail(SDPA_ERR_INVALID_ARG, "lse (the forward's statistic) is required");
  const long long rows = (long long)b * h * s_q;
  if (qwork && kwork && fixed && rows > sdpa07::kBwdFixedWorkspaceRows)
    return fail(SDPA_ERR_UNSUPPORTED,
                "%s: b * h * s_q = %lld query rows exceed the fixed workspace's %lld "
                "(use sdpa_bwd_ex with a workspace of its own)",
                what, rows, sdpa07::kBwdFixedWorkspaceRows);
  if (qwork && kwork && !fixed &&
      (st = check_workspace(workspace, workspace_bytes, rows)) != SDPA_OK)
    return st;
  const long long tq = (s_q + sdpa07::kBwdBlockM - 1) / sdpa07::kBwdBlockM;
  const long long tk = (s_kv + sdpa07::kBwdBlockN - 1) / sdpa07::kBwdBlockN;
  if ((long long)b * h * (tq > tk ? tq : tk) > 0x7fffffffLL)
    return fail(SDPA_ERR_INVALID_ARG, "grid exceeds int32");
  if (!work) return ok();
  if (fixed) {
    workspace = nullptr;
    if (qwork && kwork) {
      const hipError_t e = sdpa07::bwd_fixed_workspace(&workspace);
      if (e != hipSuccess)
        return fail(SDPA_ERR_LAUNCH, "%s: no fixed workspace on the current device: %s", what,
                    hipGetErrorString(e));
    }
  }

  sdpa07::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv; p.delta = (float*)workspace;
  p.q_sb = q_stride[0]; p.q_sh = q_stride[1]; p.q_ss = q_stride[2];
  p.k_sb = k_stride[0]; p.k_sh = k_stride[1]; p.k_ss = k_stride[2];
  p.v_sb = v_stride[0]; p.v_sh = v_stride[1]; p.v_ss = v_stride[2];
  p.o_sb = o_stride[0]; p.o_sh = o_stride[1]; p.o_ss = o_stride[2];
  p.do_sb = do_stride[0]; p.do_sh = do_stride[1]; p.do_ss = do_stride[2];
  p.dq_sb = dq_stride[0]; p.dq_sh = dq_stride[1]; p.dq_ss = dq_stride[2];
  p.dk_sb = dk_stride[0]; p.dk_sh = dk_stride[1]; p.dk_ss = dk_stride[2];
  p.dv_sb = dv_stride[0]; p.dv_sh = dv_stride[1]; p.dv_ss = dv_stride[2];
  p.b = b; p.h = h; p.s_q = s_q; p.s_kv = s_kv;
  p.h_kv = h_kv; p.bottom_right = bottom_right; p.window_left = window_left;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  if (log_enabled())
    fprintf(stderr,
            "[sdpa07] bwd dtype=%d b=%d h=%d h_kv=%d s_q=%d s_kv=%d d=%d causal=%d br=%d "
            "window=%d\n",
            (int)dtype, b, h, h_kv, s_q, s_kv, d, causal, bottom_right, window_left);
  return launch_status(
      sdpa07::launch_bwd(p, to_dt(dtype), d, causal != 0, false, (hipStream_t)stream), what);
}

}  // namespace

sdpa_status sdpa_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, sdpa_dtype dtype, int b, int h,
                        int h_kv, int s_q, int s_kv, int d, const int64_t q_stride[4],
                        const int64_t k_stride[4], const int64_t v_stride[4],
                        const int64_t o_stride[4], const int64_t do_stride[4],
                        const int64_t dq_stride[4], const int64_t dk_stride[4],
                        const int64_t dv_stride[4], float scale, int causal, int bottom_right,
                        int window_left, void* stream) {
  return bwd_dense(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, false, dtype, b,
                   h, h_kv, s_q, s_kv, d, q_stride, k_stride, v_stride, o_stride, do_stride,
                   dq_stride, dk_stride, dv_stride, scale, causal, bottom_right, window_left,
                   stream, "sdpa_bwd");
}

sdpa_status sdpa_bwd_ex_noalloc(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                sdpa_dtype dtype, int b, int h, int h_kv, int s_q, int s_kv,
                                int d, const int64_t q_stride[4], const int64_t k_stride[4],
                                const int64_t v_stride[4], const int64_t o_stride[4],
                                const int64_t do_stride[4], const int64_t dq_stride[4],
                                const int64_t dk_stride[4], const int64_t dv_stride[4],
                                float scale, int causal, int bottom_right, int window_left,
                                void* stream) {
  return bwd_dense(q, k, v, o, dout, lse, dq, dk, dv, nullptr, 0, true, dtype, b, h, h_kv, s_q,
                   s_kv, d, q_stride, k_stride, v_stride, o_stride, do_stride, dq_stride,
                   dk_stride, dv_stride, scale, causal, bottom_right, window_left, stream,
                   "sdpa_bwd_ex_noalloc");
}

sdpa_status sdpa_bwd(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes, sdpa_dtype dtype, int b, int h,
                     int s_q, int s_kv, int d, const int64_t q_stride[4],
                     const int64_t k_stride[4], const int64_t v_stride[4],
                     const int64_t o_stride[4], const int64_t do_stride[4],
                     const int64_t dq_stride[4], const int64_t dk_stride[4],
                     const int64_t dv_stride[4], float scale, int causal, void* stream) {
  return sdpa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, dtype, b, h,
                     h, s_q, s_kv, d, q_stride, k_stride, v_stride, o_stride, do_stride,
                     dq_stride, dk_stride, dv_stride, scale, causal, 0, -1, stream);
}

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
                            int bottom_right, int window_left, void* stream) {
  if (!valid_dtype(dtype)) return fail(SDPA_ERR_UNSUPPORTED, "unsupported dtype %d", (int)dtype);
  if (dtype == SDPA_FP32)
    return fail(SDPA_ERR_UNSUPPORTED, "backward supports fp16 and bf16 io only");
  if (num_seqs < 0 || total_q < 0 || total_kv < 0 || h < 0 || d < 0 || max_seqlen_q < 0 ||
      max_seqlen_kv < 0)
    return fail(SDPA_ERR_INVALID_ARG, "negative size");
  if (d != 64 && d != 128) return fail(SDPA_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d);
  if (!std::isfinite(scale)) return fail(SDPA_ERR_INVALID_ARG, "scale is not finite");
  sdpa_status st;
  if ((st = check_mask(causal, bottom_right, window_left)) != SDPA_OK) return st;
  if ((st = check_heads(h, h_kv)) != SDPA_OK) return st;
  const bool work = num_seqs > 0 && h > 0 && (total_q > 0 || total_kv > 0);
  const bool qwork = work && total_q > 0, kwork = work && total_kv > 0;
  if (work && (!cu_seqlens_q || !cu_seqlens_kv))
    return fail(SDPA_ERR_INVALID_ARG, "packed path needs cu_seqlens_q and cu_seqlens_kv");
  if ((qwork && max_seqlen_q <= 0) || (kwork && max_seqlen_kv <= 0))
    return fail(SDPA_ERR_INVALID_ARG, "packed path needs max_seqlen_q > 0 and max_seqlen_kv > 0");
  if ((work && max_seqlen_q > total_q) || (work && max_seqlen_kv > total_kv))
    return fail(SDPA_ERR_INVALID_ARG, "max_seqlen (%d, %d) exceeds the totals (%d, %d)",
                max_seqlen_q, max_seqlen_kv, total_q, total_kv);
  const int qs[3] = {total_q, h, d}, ks[3] = {total_kv, h_kv, d};
  if ((st = check_tensor("q", q, q_stride, qs, 3, dtype, qwork && kwork)) != SDPA_OK) return st;
  if ((st = check_tensor("o", o, o_stride, qs, 3, dtype, qwork && kwork)) != SDPA_OK) return st;
  if ((st = check_tensor("dout", dout, do_stride, qs, 3, dtype, qwork && kwork)) != SDPA_OK)
    return st;
  if ((st = check_tensor("dq", dq, dq_stride, qs, 3, dtype, qwork)) != SDPA_OK) return st;
  if ((st = check_tensor("k", k, k_stride, ks, 3, dtype, qwork && kwork)) != SDPA_OK) return st;
  if ((st = check_tensor("v", v, v_stride, ks, 3, dtype, qwork && kwork)) != SDPA_OK) return st;
  if ((st = check_tensor("dk", dk, dk_stride, ks, 3, dtype, kwork)) != SDPA_OK) return st;
  if ((st = check_tensor("dv", dv, dv_stride, ks, 3, dtype, kwork)) != SDPA_OK) return st;
  if ((st = check_tile_span("q", q_stride[0], dtype)) != SDPA_OK) return st;
  if ((st = check_tile_span("dout", do_stride[0], dtype)) != SDPA_OK) return st;
  if ((st = check_tile_span("k", k_stride[0], dtype)) != SDPA_OK) return st;
  if ((st = check_tile_span("v", v_stride[0], dtype)) != SDPA_OK) return st;
  if (qwork && kwork && !lse)
    return fail(SDPA_ERR_INVALID_ARG, "lse (the forward's statistic) is required");
  if (lse && reinterpret_cast<uintptr_t>(lse) % 4 != 0)
    return fail(SDPA_ERR_UNSUPPORTED, "lse: pointer is not 4-byte aligned");
  if (qwork && kwork &&
      (st = check_workspace(workspace, workspace_bytes, (long long)total_q * h)) != SDPA_OK)
    return st;
  // one workgroup per live query tile (dQ) or key tile (dK, dV) per head,
  // bounded from the totals (the kernels find their units from cu_seqlens)
  if (sdpa07::packed_units_per_head(total_q, num_seqs, sdpa07::kBwdBlockM) * h > 0x7fffffffLL ||
      sdpa07::packed_units_per_head(total_kv, num_seqs, sdpa07::kBwdBlockN) * h > 0x7fffffffLL)
    return fail(SDPA_ERR_INVALID_ARG, "grid exceeds int32");
  if (!work) return ok();

  sdpa07::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv; p.delta = (float*)workspace;
  p.q_ss = q_stride[0]; p.q_sh = q_stride[1];
  p.k_ss = k_stride[0]; p.k_sh = k_stride[1];
  p.v_ss = v_stride[0]; p.v_sh = v_stride[1];
  p.o_ss = o_stride[0]; p.o_sh = o_stride[1];
  p.do_ss = do_stride[0]; p.do_sh = do_stride[1];
  p.dq_ss = dq_stride[0]; p.dq_sh = dq_stride[1];
  p.dk_ss = dk_stride[0]; p.dk_sh = dk_stride[1];
  p.dv_ss = dv_stride[0]; p.dv_sh = dv_stride[1];
  p.b = num_seqs; p.h = h; p.s_q = max_seqlen_q; p.s_kv = max_seqlen_kv;
  p.h_kv = h_kv; p.bottom_right = bottom_right; p.window_left = window_left;
  p.cu_q = cu_seqlens_q; p.cu_kv = cu_seqlens_kv;
  p.total_q = total_q; p.total_kv = total_kv;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  if (log_enabled())
    fprintf(stderr,
            "[sdpa07] bwd_varlen dtype=%d n=%d h=%d h_kv=%d T_q=%d T_kv=%d max_q=%d max_kv=%d "
            "d=%d causal=%d br=%d window=%d\n",
            (int)dtype, num_seqs, h, h_kv, total_q, total_kv, max_seqlen_q, max_seqlen_kv, d,
            causal, bottom_right, window_left);
  return launch_status(
      sdpa07::launch_bwd(p, to_dt(dtype), d, causal != 0, true, (hipStream_t)stream),
      "sdpa_bwd_varlen");
}

sdpa_status sdpa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                         const float* descale_q, const float* descale_k, const float* descale_v,
                         const float* scale_o, float* amax_o, sdpa_dtype o_dtype, int b, int h,
                         int h_kv, int s_q, int s_kv, int d, const int64_t q_stride[4],
                         const int64_t k_stride[4], const int64_t v_stride[4],
                         const int64_t o_stride[4], float scale, int causal, int bottom_right,
                         int window_left, void* stream) {
  sdpa_status st;
  if ((st = check_fp8_extras(o_dtype, descale_q, descale_k, descale_v, scale_o, amax_o)) != SDPA_OK)
    return st;
  if (b < 0 || h < 0 || s_q < 0 || s_kv < 0 || d < 0)
    return fail(SDPA_ERR_INVALID_ARG, "negative size");
  if (d != 64 && d != 128) return fail(SDPA_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d);
  if (!std::isfinite(scale)) return fail(SDPA_ERR_INVALID_ARG, "scale is not finite");
  if ((st = check_mask(causal, bottom_right, window_left)) != SDPA_OK) return st;
  if ((st = check_heads(h, h_kv)) != SDPA_OK) return st;
  const bool work = b > 0 && h > 0 && s_q > 0;
  const int qs[4] = {b, h, s_q, d}, ks[4] = {b, h_kv, s_kv, d};
  if ((st = check_tensor("q", q, q_stride, qs, 4, SDPA_FP8_E4M3, work)) != SDPA_OK) return st;
  if ((st = check_tensor("o", o, o_stride, qs, 4, o_dtype, work)) != SDPA_OK) return st;
  if ((st = check_tensor("k", k, k_stride, ks, 4, SDPA_FP8_E4M3, work && s_kv > 0)) != SDPA_OK)
    return st;
  if ((st = check_tensor("v", v, v_stride, ks, 4, SDPA_FP8_E4M3, work && s_kv > 0)) != SDPA_OK)
    return st;
  if (lse && reinterpret_cast<uintptr_t>(lse) % 4 != 0)
    return fail(SDPA_ERR_UNSUPPORTED, "lse: pointer is not 4-byte aligned");
  const long long n_qtiles = (s_q + sdpa07::kFwdBlockM - 1) / sdpa07::kFwdBlockM;
  if ((long long)b * h * n_qtiles > 0x7fffffffLL)
    return fail(SDPA_ERR_INVALID_ARG, "grid exceeds int32");
  if (!work) return ok();

  sdpa07::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.q_sb = q_stride[0]; p.q_sh = q_stride[1]; p.q_ss = q_stride[2];
  p.k_sb = k_stride[0]; p.k_sh = k_stride[1]; p.k_ss = k_stride[2];
  p.v_sb = v_stride[0]; p.v_sh = v_stride[1]; p.v_ss = v_stride[2];
  p.o_sb = o_stride[0]; p.o_sh = o_stride[1]; p.o_ss = o_stride[2];
  p.b = b; p.h = h; p.h_kv = h_kv; p.s_q = s_q; p.s_kv = s_kv;
  p.bottom_right = bottom_right; p.window_left = window_left;
  p.n_qtiles = (int)n_qtiles;
  p.scale = scale;
  p.descale_q = descale_q; p.descale_k = descale_k; p.descale_v = descale_v;
  p.scale_o = scale_o; p.amax_o = amax_o;
  if (log_enabled())
    fprintf(stderr,
            "[sdpa07] fwd_fp8 out=%d b=%d h=%d h_kv=%d s_q=%d s_kv=%d d=%d causal=%d br=%d "
            "window=%d\n",
            (int)o_dtype, b, h, h_kv, s_q, s_kv, d, causal, bottom_right, window_left);
  return launch_status(sdpa07::launch_fwd_fp8(p, to_dt(o_dtype), d, causal != 0, false,
                                              (hipStream_t)stream),
                       "sdpa_fwd_fp8");
}

sdpa_status sdpa_fwd_fp8_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                const float* descale_q, const float* descale_k,
                                const float* descale_v, const float* scale_o, float* amax_o,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                int num_seqs, int total_q, int total_kv, int max_seqlen_q,
                                int max_seqlen_kv, sdpa_dtype o_dtype, int h, int h_kv, int d,
                                const int64_t q_stride[3], const int64_t k_stride[3],
                                const int64_t v_stride[3], const int64_t o_stride[3],
                                float scale, int causal, int bottom_right, int window_left,
                                void* stream) {
  sdpa_status st;
  if ((st = check_fp8_extras(o_dtype, descale_q, descale_k, descale_v, scale_o, amax_o)) != SDPA_OK)
    return st;
  if (num_seqs < 0 || total_q < 0 || total_kv < 0 || h < 0 || d < 0 || max_seqlen_q < 0 ||
      max_seqlen_kv < 0)
    return fail(SDPA_ERR_INVALID_ARG, "negative size");
  if (d != 64 && d != 128) return fail(SDPA_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d);
  if (!std::isfinite(scale)) return fail(SDPA_ERR_INVALID_ARG, "scale is not finite");
  if ((st = check_mask(causal, bottom_right, window_left)) != SDPA_OK) return st;
  if ((st = check_heads(h, h_kv)) != SDPA_OK) return st;
  const bool work = num_seqs > 0 && h > 0 && total_q > 0;
  if (work && (!cu_seqlens_q || !cu_seqlens_kv))
    return fail(SDPA_ERR_INVALID_ARG, "packed path needs cu_seqlens_q and cu_seqlens_kv");
  if (work && (max_seqlen_q <= 0 || max_seqlen_kv <= 0))
    return fail(SDPA_ERR_INVALID_ARG, "packed path needs max_seqlen_q > 0 and max_seqlen_kv > 0");
  if (work && max_seqlen_q > total_q)
    return fail(SDPA_ERR_INVALID_ARG, "max_seqlen_q %d exceeds total_q %d", max_seqlen_q,
                total_q);
  const int qs[3] = {total_q, h, d}, ks[3] = {total_kv, h_kv, d};
  if ((st = check_tensor("q", q, q_stride, qs, 3, SDPA_FP8_E4M3, work)) != SDPA_OK) return st;
  if ((st = check_tensor("o", o, o_stride, qs, 3, o_dtype, work)) != SDPA_OK) return st;
  if ((st = check_tensor("k", k, k_stride, ks, 3, SDPA_FP8_E4M3, work && total_kv > 0)) != SDPA_OK)
    return st;
  if ((st = check_tensor("v", v, v_stride, ks, 3, SDPA_FP8_E4M3, work && total_kv > 0)) != SDPA_OK)
    return st;
  if (lse && reinterpret_cast<uintptr_t>(lse) % 4 != 0)
    return fail(SDPA_ERR_UNSUPPORTED, "lse: pointer is not 4-byte aligned");
  const long long n_qtiles = (max_seqlen_q + sdpa07::kFwdBlockM - 1) / sdpa07::kFwdBlockM;
  // one workgroup per live query tile (or pair of tiles) per head, bounded
  // from the totals (the kernels find their units from cu_seqlens)
  if (sdpa07::packed_units_per_head(total_q, num_seqs, sdpa07::kFwdBlockM) * h > 0x7fffffffLL)
    return fail(SDPA_ERR_INVALID_ARG, "grid exceeds int32");
  if (!work) return ok();

  sdpa07::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.q_ss = q_stride[0]; p.q_sh = q_stride[1];
  p.k_ss = k_stride[0]; p.k_sh = k_stride[1];
  p.v_ss = v_stride[0]; p.v_sh = v_stride[1];
  p.o_ss = o_stride[0]; p.o_sh = o_stride[1];
  p.b = num_seqs; p.h = h; p.h_kv = h_kv;
  p.bottom_right = bottom_right; p.window_left = window_left;
  p.n_qtiles = (int)n_qtiles;
  p.cu_q = cu_seqlens_q; p.cu_kv = cu_seqlens_kv;
  p.total_q = total_q; p.total_kv = total_kv;
  p.scale = scale;
  p.descale_q = descale_q; p.descale_k = descale_k; p.descale_v = descale_v;
  p.scale_o = scale_o; p.amax_o = amax_o;
  if (log_enabled())
    fprintf(stderr,
            "[sdpa07] fwd_fp8_varlen out=%d n=%d h=%d h_kv=%d T_q=%d T_kv=%d max_q=%d d=%d "
            "causal=%d br=%d window=%d\n",
            (int)o_dtype, num_seqs, h, h_kv, total_q, total_kv, max_seqlen_q, d, causal,
            bottom_right, window_left);
  return launch_status(sdpa07::launch_fwd_fp8(p, to_dt(o_dtype), d, causal != 0, true,
                                              (hipStream_t)stream),
                       "sdpa_fwd_fp8_varlen");
}

}  // extern "C"
