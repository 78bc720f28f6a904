// Oracle for scaled-dot-product attention: a plain, slow, fp64 CPU
// implementation of the definition. TEST INFRASTRUCTURE ONLY.
//
// Only tests/, the smoke check and the benchmark's CPU-baseline leg load
// this library. It shares no code, header or constant with the GPU library,
// and the GPU library never calls it.
//
// What it computes (no blocking, no online softmax, no reordering beyond the
// definition):
//   O = softmax(scale * Q K^T + mask) V, row by row, in double precision,
//   LSE_i = log sum_j exp(scale * q_i . k_j) over the visible keys j (natural
//   log, scale included), and the backward quantities dQ, dK, dV.
//
// Sources (page titles and sections; the pages state no formula, so the
// textbook definition is used where they name the operation):
//  * "Inside NVIDIA's cuDNN Graph API: Fusion, Autotuning, and Plan Reuse
//    with cuDNN Frontend", section 5 "SDPA (Flash Attention) with causal
//    masking": the operation, its attention scale, causal masking given as a
//    top-left diagonal band with right bound 0 (key j visible to query i iff
//    j <= i), and torch's scaled_dot_product_attention as the check.
//  * cudnn-frontend pull request #554 "torch: put torch.sdpa on the cuDNN
//    Python API (CUDNN provider + dense backward)": the forward returns the
//    per-row statistics in aten's logsumexp layout (B, H, S) fp32 for dense
//    and token-major (T, H) for packed THD; the packed path is indexed by
//    cu_seqlens prefix sums with no attention across sequences; the dense
//    backward returns dQ, dK, dV from Q, K, V, O, dO and the statistics.
//  * The same pull request's merge log, the entry converting the SM80
//    backward to a TemplateParams module: the backward chain starts with a
//    row dot product of dO and O (the "do_dot" step).
//  * The same merge log, the entry adding the d512 FP8 forward: a query row
//    with no visible key is a dead row whose statistic is -inf and whose
//    output comes from an all-zero P; a zero-length sequence contributes
//    nothing.
//
//  * The same merge log, the per-tensor FP8 forward entry: e4m3 inputs with
//    per-tensor descales; oracle_e4m3_decode gives their exact values (the
//    bit layout is the public OCP FP8 one, stated at the function).
//  * The same pull request's sdpa API: is_causal (top-left), causal_bottom_right
//    (the diagonal aligned to the bottom-right corner, allowed only with an
//    active band) and window_left (-1 = unbounded), and grouped-query
//    attention (h_kv < h_q) served by the provider; its dense-backward tests
//    note that GQA dK/dV sum over the h_q/h_kv query heads of a group.
//
// Readings taken where the pages are silent: causal is top-left even when
// s_q != s_kv; bottom-right aligns query i with key i + s_kv - s_q (per
// sequence in packed batches); window_left = W keeps the W keys left of the
// aligned diagonal and the diagonal key itself (keys j >= p - W, inclusive),
// and without causal only that left bound applies; query head hh reads K/V
// head hh / (h_q / h_kv); a row with no visible key gets O = 0 and LSE =
// -inf; nothing is rounded (the GPU's rounding of P and of outputs is
// absorbed by tolerances).
//
// Layouts (all contiguous, row-major, double):
//   dense : q, o [b][h][s_q][d]; k, v [b][h][s_kv][d]; lse [b][h][s_q]
//   varlen: q, o [total_q][h][d]; k, v [total_kv][h][d]; lse [total_q][h]

#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>
#include <algorithm>
#include <functional>

namespace {

// Run fn(i) for i in [0, n) over `threads` std::threads, contiguous chunks.
void parallel_for(int64_t n, int threads, const std::function<void(int64_t)>& fn) {
  if (n <= 0) return;
  if (threads <= 0) threads = (int)std::max(1u, std::thread::hardware_concurrency());
  if (threads > n) threads = (int)n;
  if (threads == 1) {
    for (int64_t i = 0; i < n; ++i) fn(i);
    return;
  }
  std::vector<std::thread> pool;
  int64_t chunk = (n + threads - 1) / threads;
  for (int t = 0; t < threads; ++t) {
    int64_t lo = t * chunk, hi = std::min(n, lo + chunk);
    if (lo >= hi) break;
    pool.emplace_back([lo, hi, &fn] { for (int64_t i = lo; i < hi; ++i) fn(i); });
  }
  for (auto& th : pool) th.join();
}

// The mask options of one call (the sdpa API of cudnn-frontend PR #554).
struct Mask {
  int causal;        // right bound 0 on the aligned diagonal
  int bottom_right;  // align the diagonal with the bottom-right corner
  int64_t window;    // window_left; < 0: no left bound
};

// Key j is visible to the query at position i of a (s_q, s_kv) problem
// (cuDNN frontend demo, section 5: causal = diagonal band with right bound 0,
// aligned top-left; PR #554's sdpa: bottom-right alignment, window_left).
inline bool visible(int64_t i, int64_t j, int64_t s_q, int64_t s_kv, const Mask& m) {
  const int64_t p = m.bottom_right ? i + s_kv - s_q : i;  // diagonal key of row i
  if (m.causal && j > p) return false;
  if (m.window >= 0 && j < p - m.window) return false;
  return true;
}

// One query row against one head's keys: the definition of softmax attention.
// q: [d]; k, v: [s_kv][d] with row stride `kv_stride` elements; o: [d].
void attend_row(const double* q, int64_t pos, int64_t s_q, const double* k, const double* v,
                int64_t kv_stride, int64_t s_kv, int64_t d, double scale, const Mask& mask,
                double* o, double* lse) {
  std::vector<double> x(s_kv > 0 ? s_kv : 1);
  double m = -std::numeric_limits<double>::infinity();
  int64_t n_vis = 0;
  for (int64_t j = 0; j < s_kv; ++j) {
    if (!visible(pos, j, s_q, s_kv, mask)) continue;
    double dot = 0.0;
    for (int64_t c = 0; c < d; ++c) dot += q[c] * k[j * kv_stride + c];
    x[j] = scale * dot;
    m = std::max(m, x[j]);
    ++n_vis;
  }
  for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
  if (n_vis == 0) {  // dead row: empty softmax, zero output
    *lse = -std::numeric_limits<double>::infinity();
    return;
  }
  double l = 0.0;
  for (int64_t j = 0; j < s_kv; ++j)
    if (visible(pos, j, s_q, s_kv, mask)) l += std::exp(x[j] - m);
  const double L = m + std::log(l);
  *lse = L;
  for (int64_t j = 0; j < s_kv; ++j) {
    if (!visible(pos, j, s_q, s_kv, mask)) continue;
    const double p = std::exp(x[j] - L);
    for (int64_t c = 0; c < d; ++c) o[c] += p * v[j * kv_stride + c];
  }
}

// Backward of one query head, given that head's forward O and LSE (fp64).
// Row strides let the same routine serve dense (stride d) and packed THD
// (stride h*d) heads. dQ is written; dK and dV are ADDED to (a K/V head
// collects the contributions of every query head of its group).
void backward_head(const double* q, const double* k, const double* v, const double* o,
                   const double* dout, const double* lse, int64_t qs, int64_t ks,
                   int64_t s_q, int64_t s_kv, int64_t d, double scale, const Mask& mask,
                   double* dq, double* dk, double* dv, int threads) {
  // P and dS as full [s_q][s_kv] matrices (zero where the key is hidden).
  std::vector<double> P((size_t)(s_q * s_kv)), dS((size_t)(s_q * s_kv));
  parallel_for(s_q, threads, [&](int64_t i) {
    const double* qi = q + i * qs;
    const double* gi = dout + i * qs;
    const double* oi = o + i * qs;
    double D = 0.0;  // rowsum(dO * O)
    for (int64_t c = 0; c < d; ++c) D += gi[c] * oi[c];
    for (int64_t j = 0; j < s_kv; ++j) {
      double p = 0.0, ds = 0.0;
      if (visible(i, j, s_q, s_kv, mask) && std::isfinite(lse[i])) {
        double dot = 0.0, dp = 0.0;
        for (int64_t c = 0; c < d; ++c) {
          dot += qi[c] * k[j * ks + c];
          dp += gi[c] * v[j * ks + c];
        }
        p = std::exp(scale * dot - lse[i]);
        ds = p * (dp - D);
      }
      P[(size_t)(i * s_kv + j)] = p;
      dS[(size_t)(i * s_kv + j)] = ds;
    }
  });
  // dQ_i = scale * sum_j dS_ij k_j
  parallel_for(s_q, threads, [&](int64_t i) {
    for (int64_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int64_t j = 0; j < s_kv; ++j) acc += dS[(size_t)(i * s_kv + j)] * k[j * ks + c];
      dq[i * qs + c] = scale * acc;
    }
  });
  // dK_j = scale * sum_i dS_ij q_i ; dV_j = sum_i P_ij dO_i
  parallel_for(s_kv, threads, [&](int64_t j) {
    for (int64_t c = 0; c < d; ++c) {
      double ak = 0.0, av = 0.0;
      for (int64_t i = 0; i < s_q; ++i) {
        ak += dS[(size_t)(i * s_kv + j)] * q[i * qs + c];
        av += P[(size_t)(i * s_kv + j)] * dout[i * qs + c];
      }
      dk[j * ks + c] += scale * ak;
      dv[j * ks + c] += av;
    }
  });
}

}  // namespace

extern "C" {

int oracle_hardware_threads(void) {
  return (int)std::max(1u, std::thread::hardware_concurrency());
}

// Selected query rows of one head: row r of q sits at position q_pos[r] of a
// problem with s_q query rows and attends to the s_kv rows of k, v.
// q, o: [n_q][d]; k, v: [s_kv][d]; lse: [n_q].
void oracle_attn_rows_ex(const double* q, const int64_t* q_pos, int64_t n_q, int64_t s_q,
                         const double* k, const double* v, int64_t s_kv, int64_t d, double scale,
                         int causal, int bottom_right, int64_t window, double* o, double* lse,
                         int threads) {
  const Mask mask{causal, bottom_right, window};
  parallel_for(n_q, threads, [&](int64_t r) {
    attend_row(q + r * d, q_pos[r], s_q, k, v, d, s_kv, d, scale, mask, o + r * d, lse + r);
  });
}

void oracle_attn_rows(const double* q, const int64_t* q_pos, int64_t n_q, const double* k,
                      const double* v, int64_t s_kv, int64_t d, double scale, int causal,
                      double* o, double* lse, int threads) {
  oracle_attn_rows_ex(q, q_pos, n_q, 0, k, v, s_kv, d, scale, causal, 0, -1, o, lse, threads);
}

// Dense forward, BHSD contiguous; q, o have h_q heads, k, v have h_kv heads
// (h_q a multiple of h_kv).
void oracle_fwd_ex(const double* q, const double* k, const double* v, int64_t b, int64_t h_q,
                   int64_t h_kv, int64_t s_q, int64_t s_kv, int64_t d, double scale, int causal,
                   int bottom_right, int64_t window, double* o, double* lse, int threads) {
  const Mask mask{causal, bottom_right, window};
  const int64_t group = h_q / h_kv;
  parallel_for(b * h_q * s_q, threads, [&](int64_t r) {
    const int64_t bh = r / s_q, i = r % s_q;
    const int64_t bi = bh / h_q, hq = bh % h_q;
    const int64_t kvo = (bi * h_kv + hq / group) * s_kv * d;
    attend_row(q + r * d, i, s_q, k + kvo, v + kvo, d, s_kv, d, scale, mask, o + r * d, lse + r);
  });
}

void oracle_fwd(const double* q, const double* k, const double* v, int64_t b, int64_t h,
                int64_t s_q, int64_t s_kv, int64_t d, double scale, int causal, double* o,
                double* lse, int threads) {
  oracle_fwd_ex(q, k, v, b, h, h, s_q, s_kv, d, scale, causal, 0, -1, o, lse, threads);
}

// Packed THD forward. Sequence n owns tokens [cu_q[n], cu_q[n+1]) of q and
// [cu_kv[n], cu_kv[n+1]) of k, v; positions are local to the sequence.
// q, o: [T_q][h_q][d]; k, v: [T_kv][h_kv][d]; lse: [T_q][h_q].
void oracle_fwd_varlen_ex(const double* q, const double* k, const double* v, const int32_t* cu_q,
                          const int32_t* cu_kv, int64_t n_seqs, int64_t h_q, int64_t h_kv,
                          int64_t d, double scale, int causal, int bottom_right, int64_t window,
                          double* o, double* lse, int threads) {
  const Mask mask{causal, bottom_right, window};
  const int64_t group = h_q / h_kv;
  const int64_t total_q = n_seqs > 0 ? cu_q[n_seqs] : 0;
  parallel_for(total_q * h_q, threads, [&](int64_t r) {
    const int64_t t = r / h_q, hh = r % h_q;
    int64_t n = 0;
    while (n + 1 < n_seqs && cu_q[n + 1] <= t) ++n;  // sequence owning token t
    const int64_t pos = t - cu_q[n], s_q = cu_q[n + 1] - cu_q[n];
    const int64_t kv0 = cu_kv[n], s_kv = cu_kv[n + 1] - cu_kv[n];
    const int64_t kvo = (kv0 * h_kv + hh / group) * d;
    attend_row(q + (t * h_q + hh) * d, pos, s_q, k + kvo, v + kvo, h_kv * d, s_kv, d, scale,
               mask, o + (t * h_q + hh) * d, lse + t * h_q + hh);
  });
}

void oracle_fwd_varlen(const double* q, const double* k, const double* v, const int32_t* cu_q,
                       const int32_t* cu_kv, int64_t n_seqs, int64_t h, int64_t d, double scale,
                       int causal, double* o, double* lse, int threads) {
  oracle_fwd_varlen_ex(q, k, v, cu_q, cu_kv, n_seqs, h, h, d, scale, causal, 0, -1, o, lse,
                       threads);
}

// Dense backward, BHSD contiguous (heads as in oracle_fwd_ex). Runs its own
// fp64 forward for O and LSE (returned in o and lse), then the backward of
// every query head; a K/V head's dK and dV sum over its group.
void oracle_bwd_ex(const double* q, const double* k, const double* v, const double* dout,
                   int64_t b, int64_t h_q, int64_t h_kv, int64_t s_q, int64_t s_kv, int64_t d,
                   double scale, int causal, int bottom_right, int64_t window, double* o,
                   double* lse, double* dq, double* dk, double* dv, int threads) {
  const Mask mask{causal, bottom_right, window};
  const int64_t group = h_q / h_kv;
  oracle_fwd_ex(q, k, v, b, h_q, h_kv, s_q, s_kv, d, scale, causal, bottom_right, window, o, lse,
                threads);
  std::memset(dk, 0, sizeof(double) * (size_t)(b * h_kv * s_kv * d));
  std::memset(dv, 0, sizeof(double) * (size_t)(b * h_kv * s_kv * d));
  for (int64_t bh = 0; bh < b * h_q; ++bh) {
    const int64_t bi = bh / h_q, hq = bh % h_q;
    const int64_t qo = bh * s_q * d, ko = (bi * h_kv + hq / group) * s_kv * d;
    backward_head(q + qo, k + ko, v + ko, o + qo, dout + qo, lse + bh * s_q, d, d, s_q, s_kv, d,
                  scale, mask, dq + qo, dk + ko, dv + ko, threads);
  }
}

void oracle_bwd(const double* q, const double* k, const double* v, const double* dout,
                int64_t b, int64_t h, int64_t s_q, int64_t s_kv, int64_t d, double scale,
                int causal, double* o, double* lse, double* dq, double* dk, double* dv,
                int threads) {
  oracle_bwd_ex(q, k, v, dout, b, h, h, s_q, s_kv, d, scale, causal, 0, -1, o, lse, dq, dk, dv,
                threads);
}

// Packed THD backward, same conventions as oracle_fwd_varlen_ex.
void oracle_bwd_varlen_ex(const double* q, const double* k, const double* v, const double* dout,
                          const int32_t* cu_q, const int32_t* cu_kv, int64_t n_seqs, int64_t h_q,
                          int64_t h_kv, int64_t d, double scale, int causal, int bottom_right,
                          int64_t window, double* o, double* lse, double* dq, double* dk,
                          double* dv, int threads) {
  const Mask mask{causal, bottom_right, window};
  const int64_t group = h_q / h_kv;
  oracle_fwd_varlen_ex(q, k, v, cu_q, cu_kv, n_seqs, h_q, h_kv, d, scale, causal, bottom_right,
                       window, o, lse, threads);
  const int64_t total_kv = n_seqs > 0 ? cu_kv[n_seqs] : 0;
  std::memset(dk, 0, sizeof(double) * (size_t)(total_kv * h_kv * d));
  std::memset(dv, 0, sizeof(double) * (size_t)(total_kv * h_kv * d));
  for (int64_t n = 0; n < n_seqs; ++n) {
    const int64_t q0 = cu_q[n], sq = cu_q[n + 1] - cu_q[n];
    const int64_t k0 = cu_kv[n], skv = cu_kv[n + 1] - cu_kv[n];
    if (sq == 0 && skv == 0) continue;
    // lse is [t][h_q]: gather one head's column for this sequence.
    for (int64_t hh = 0; hh < h_q; ++hh) {
      std::vector<double> lse_h((size_t)std::max<int64_t>(sq, 1));
      for (int64_t i = 0; i < sq; ++i) lse_h[(size_t)i] = lse[(q0 + i) * h_q + hh];
      const int64_t qo = (q0 * h_q + hh) * d, ko = (k0 * h_kv + hh / group) * d;
      backward_head(q + qo, k + ko, v + ko, o + qo, dout + qo, lse_h.data(), h_q * d, h_kv * d,
                    sq, skv, d, scale, mask, dq + qo, dk + ko, dv + ko, threads);
    }
  }
}

void oracle_bwd_varlen(const double* q, const double* k, const double* v, const double* dout,
                       const int32_t* cu_q, const int32_t* cu_kv, int64_t n_seqs, int64_t h,
                       int64_t d, double scale, int causal, double* o, double* lse, double* dq,
                       double* dk, double* dv, int threads) {
  oracle_bwd_varlen_ex(q, k, v, dout, cu_q, cu_kv, n_seqs, h, h, d, scale, causal, 0, -1, o, lse,
                       dq, dk, dv, threads);
}

// FP8 E4M3 codes to doubles, exactly. The pages name the format (the
// per-tensor FP8 forward of cudnn-frontend PR #554's merge log runs on
// E4M3/E5M2 inputs) but not its bits; the encoding is the public OCP 8-bit
// floating point one, in the variant without infinities that the e4m3
// tensors of torch and the gfx950 conversions use: sign bit 7, exponent
// bits 6..3 with bias 7, mantissa bits 2..0; exponent field 0 holds the
// subnormals m/8 * 2^-6; exponent 15 with mantissa 7 is NaN (so the largest
// finite value is 1.75 * 2^8 = 448).
void oracle_e4m3_decode(const uint8_t* codes, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) {
    const int c = codes[i];
    const int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double x;
    if (e == 15 && m == 7)
      x = std::nan("");
    else if (e == 0)
      x = std::ldexp((double)m, -9);  // (m / 8) * 2^-6
    else
      x = std::ldexp((double)(8 + m), e - 10);  // (1 + m / 8) * 2^(e - 7)
    out[i] = sign ? -x : x;
  }
}

}  // extern "C"
