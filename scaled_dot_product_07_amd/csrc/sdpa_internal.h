// Internal interface between the C-ABI layer (abi.cpp) and the HIP kernels.
// Not installed; the public interface is include/sdpa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa07 {

enum class Dt : int { F32 = 0, F16 = 1, BF16 = 2 };

// Forward launch parameters. Strides are in elements; the d stride is 1.
// Dense: index (b, h, s). Packed THD: the "b" index is the sequence, the
// b strides are unused and rows start at cu_seqlens[n].
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int b;          // batch (dense) or number of sequences (packed)
  int h;          // query heads
  int h_kv;       // key/value heads (h is a multiple; query head i reads K/V head i / (h / h_kv))
  int s_q, s_kv;  // dense lengths (unused when packed)
  int bottom_right;  // 1: the diagonal of the band is aligned to the bottom-right corner
  int window_left;   // keys kept left of the diagonal; < 0: no left bound
  int n_qtiles;   // query tiles per (b, h): ceil(s_q or max_seqlen_q / BM)
  float scale_log2;  // |scale| * log2(e)
  int negate_q;      // 1 when scale < 0 (the sign is moved onto Q, exactly)
  const int32_t* cu_q;
  const int32_t* cu_kv;
  int total_q, total_kv;
  // fp8 (e4m3) inputs only: per-tensor factors read on the device (null
  // means 1): real Q = descale_q * Q, likewise K and V; O is stored as
  // scale_o * O. amax_o (may be null) receives max |stored O| before the
  // output cast. scale is the signed attention scale (the kernel folds it
  // with the descales into its log2 factor).
  const float* descale_q;
  const float* descale_k;
  const float* descale_v;
  const float* scale_o;
  float* amax_o;
  float scale;
  // fp16/bf16 forward: units per round of the one-tile grid (the device's
  // compute-unit count; set by the launcher)
  int split_round;
};

// Backward launch parameters (dense).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // workspace: rowsum(dO * O), fp32 [b][h][s_q]; then LSE * log2(e)
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int64_t do_sb, do_sh, do_ss;
  int64_t dq_sb, dq_sh, dq_ss;
  int64_t dk_sb, dk_sh, dk_ss;
  int64_t dv_sb, dv_sh, dv_ss;
  int b, h, s_q, s_kv;  // packed layout: b = sequences, s_q / s_kv = longest sequence
  int h_kv;             // key/value heads (h is a multiple)
  int bottom_right;     // diagonal aligned to the bottom-right corner
  int window_left;      // -1: no left bound
  float scale;          // the signed attention scale
  float scale_log2;     // scale * log2(e)
  // packed (THD) layout only: sequence starts (b + 1 entries) and totals;
  // row strides are the *_ss fields, *_sb unused
  const int32_t* cu_q;
  const int32_t* cu_kv;
  int total_q, total_kv;
};

constexpr int kFwdBlockM = 128;  // query rows per workgroup (32 per wave)
constexpr int kFwdBlockN = 64;   // keys per K/V tile
constexpr int kFwdThreads = 256;    // fp32 forward workgroup
// fp16/bf16 forward workgroup: 4 waves over one query tile at d = 64 and
// for causal bands, 8 waves over a pair of tiles sharing one key stream for
// non-causal d = 128
constexpr int kFwdThreads16 = 256;
constexpr int kFwdThreads16Pair = 512;
constexpr int fwd16_threads(int d, bool causal) {
  return d <= 64 || causal ? kFwdThreads16 : kFwdThreads16Pair;
}

// Workgroups per head of a packed (THD) launch whose units hold unit_rows
// query rows of one sequence (a 128-row tile, or a pair of them): every split
// of total rows into num_seqs sequences has at most total / unit_rows +
// num_seqs such units, so the grid needs no lengths from the device.
constexpr long long packed_units_per_head(long long total, long long num_seqs, int unit_rows) {
  return total / unit_rows + num_seqs;
}

// Enqueue the forward; returns the launch status.
// compute units of the current device (cached per device; 0 on error)
int compute_units();

hipError_t launch_fwd(const FwdParams& p, Dt dt, int d, bool causal, bool varlen,
                      hipStream_t stream);

// Enqueue the fp8 (e4m3) forward; `out` is the output dtype (F16 or BF16).
hipError_t launch_fwd_fp8(const FwdParams& p, Dt out, int d, bool causal, bool varlen,
                          hipStream_t stream);

// Enqueue the three backward kernels; returns the first failing launch status.
hipError_t launch_bwd(const BwdParams& p, Dt dt, int d, bool causal, bool varlen,
                      hipStream_t stream);

// Bytes of backward workspace for `rows` = b * h * s_q (dense) or total_q * h
// (packed) query rows: the fp32
// row dot products rowsum(dO * O) and the statistic in base 2.
size_t bwd_workspace_bytes(long long rows);

// Backward workspace held in the library's own device code, for the entry
// point that allocates nothing: 16 MiB on every device the library runs on,
// enough for bwd_workspace_bytes(2^21 query rows).
constexpr size_t kBwdFixedWorkspaceBytes = size_t(16) << 20;
constexpr long long kBwdFixedWorkspaceRows = 1LL << 21;
static_assert(kBwdFixedWorkspaceRows * 2 * sizeof(float) == kBwdFixedWorkspaceBytes,
              "two fp32 values per query row");

// Device address of the current device's copy of that workspace (looked up
// once per device, then cached).
hipError_t bwd_fixed_workspace(void** ptr);

// Tile sizes of the dK/dV and dQ passes (for grid-size validation).
constexpr int kBwdBlockM = 128;
constexpr int kBwdBlockN = 128;

}  // namespace sdpa07
