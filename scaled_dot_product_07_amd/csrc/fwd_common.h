// Forward helpers shared by the fp16/bf16/fp32 kernels (fwd.hip) and the
// fp8 kernel (fwd_fp8.hip): work-unit decoding, the band mask on the S^T
// accumulator layout and the per-tile online softmax.
#pragma once

#include "kernel_common.h"
#include "sdpa_internal.h"

namespace sdpa07 {
namespace {

// Decoded work unit of one workgroup.
struct Unit {
  int qt;          // query tile
  int hi;          // head
  int q_len, kv_len;
  int64_t q_off, k_off, v_off, o_off;  // element offsets of row 0 of this (b|seq, h)
  int64_t lse_off, lse_st;
};

// Dense: blockIdx -> (query tile, b*h) with the heaviest causal tiles first.
// Packed: blockIdx -> (live tile of a sequence, head), heads innermost; the
// tiles of all sequences come in decreasing order of work (a causal band
// without a left bound: tile t of a sequence costs t + 1 key blocks; other
// masks: its key count), a rank past the last tile gives q_len = 0.
template <bool VARLEN, bool CAUSAL>
__device__ __forceinline__ Unit decode_unit(const FwdParams& p) {
  Unit w;
  if constexpr (VARLEN) {
    w.hi = blockIdx.x % p.h;
    const bool taper = CAUSAL && p.window_left < 0;
    const PackedUnit pu = packed_unit(blockIdx.x / p.h, p.b, taper, [&](int s) -> int2 {
      const int nq = (packed_len(p.cu_q, s, p.total_q) + kFwdBlockM - 1) / kFwdBlockM;
      if (taper) return int2{nq, nq};
      const int nk = (packed_len(p.cu_kv, s, p.total_kv) + kFwdBlockN - 1) / kFwdBlockN;
      return int2{nq, max(nk, 1)};
    });
    if (pu.seq < 0) {
      w.qt = 0;
      w.q_len = 0;  // no tile: the workgroup exits
      return w;
    }
    const int bi = pu.seq;
    const int q0 = min(max(p.cu_q[bi], 0), p.total_q);
    const int q1 = min(max(p.cu_q[bi + 1], 0), p.total_q);
    const int k0 = min(max(p.cu_kv[bi], 0), p.total_kv);
    const int k1 = min(max(p.cu_kv[bi + 1], 0), p.total_kv);
    w.q_len = max(q1 - q0, 0);
    w.kv_len = max(k1 - k0, 0);
    const int nq = (w.q_len + kFwdBlockM - 1) / kFwdBlockM;
    w.qt = taper ? nq - 1 - pu.j : pu.j;
    w.q_off = (int64_t)q0 * p.q_ss + (int64_t)w.hi * p.q_sh;
    w.o_off = (int64_t)q0 * p.o_ss + (int64_t)w.hi * p.o_sh;
    w.k_off = (int64_t)k0 * p.k_ss + (int64_t)(w.hi / (p.h / p.h_kv)) * p.k_sh;
    w.v_off = (int64_t)k0 * p.v_ss + (int64_t)(w.hi / (p.h / p.h_kv)) * p.v_sh;
    w.lse_off = (int64_t)q0 * p.h + w.hi;
    w.lse_st = p.h;
  } else {
    const int nbh = p.b * p.h;
    const int u = blockIdx.x;
    w.qt = p.n_qtiles - 1 - u / nbh;  // heaviest causal tiles first
    const int bh = u % nbh;
    const int bi = bh / p.h;
    w.hi = bh % p.h;
    w.q_len = p.s_q;
    w.kv_len = p.s_kv;
    w.q_off = (int64_t)bi * p.q_sb + (int64_t)w.hi * p.q_sh;
    w.o_off = (int64_t)bi * p.o_sb + (int64_t)w.hi * p.o_sh;
    w.k_off = (int64_t)bi * p.k_sb + (int64_t)(w.hi / (p.h / p.h_kv)) * p.k_sh;
    w.v_off = (int64_t)bi * p.v_sb + (int64_t)(w.hi / (p.h / p.h_kv)) * p.v_sh;
    w.lse_off = ((int64_t)bi * p.h + w.hi) * p.s_q;
    w.lse_st = 1;
  }
  return w;
}

// One query tile per workgroup, the two tiles of a pair on one CU: the grid
// runs in rounds of 2R workgroups (R = p.split_round, the compute-unit
// count); in a round, workgroup j < R takes the first tile of the round's
// pair unit j and workgroup R + j its second, the two that the dispatcher
// places on one CU when the round is resident. Pairs: (n-1-i, i) for a
// causal band without a left bound (equal work), (2i, 2i+1) otherwise.
// Dense: unit -> (pair, b*h). Packed: unit -> (live pair of a sequence,
// head), heads innermost, pairs of all sequences heaviest first. A
// workgroup without a tile (the missing second tile of an odd count, or a
// unit past the last pair) gets q_len = 0.
template <bool VARLEN, bool CAUSAL>
__device__ __forceinline__ Unit decode_unit_paired(const FwdParams& p) {
  const int n_units = gridDim.x / 2;
  const int R = p.split_round;
  const int r = blockIdx.x / (2 * R);
  const int rem = min(R, n_units - r * R);  // units in this round
  const int off = blockIdx.x - r * 2 * R;
  const int half = off / rem;
  const int unit = r * R + off % rem;
  const bool heavy = CAUSAL && p.window_left < 0;
  Unit w;
  int pair, n_qt;
  if constexpr (VARLEN) {
    w.hi = unit % p.h;
    const PackedUnit pu = packed_unit(unit / p.h, p.b, heavy, [&](int s) -> int2 {
      const int lq = packed_len(p.cu_q, s, p.total_q);
      const int np = (lq + 2 * kFwdBlockM - 1) / (2 * kFwdBlockM);
      if (heavy) return int2{np, (lq + kFwdBlockM - 1) / kFwdBlockM};
      return int2{np, max((packed_len(p.cu_kv, s, p.total_kv) + kFwdBlockN - 1) / kFwdBlockN, 1)};
    });
    if (pu.seq < 0) {
      w.qt = 0;
      w.q_len = 0;
      return w;
    }
    const int bi = pu.seq;
    const int q0 = min(max(p.cu_q[bi], 0), p.total_q);
    const int q1 = min(max(p.cu_q[bi + 1], 0), p.total_q);
    const int k0 = min(max(p.cu_kv[bi], 0), p.total_kv);
    const int k1 = min(max(p.cu_kv[bi + 1], 0), p.total_kv);
    w.q_len = max(q1 - q0, 0);
    w.kv_len = max(k1 - k0, 0);
    w.q_off = (int64_t)q0 * p.q_ss + (int64_t)w.hi * p.q_sh;
    w.o_off = (int64_t)q0 * p.o_ss + (int64_t)w.hi * p.o_sh;
    w.k_off = (int64_t)k0 * p.k_ss + (int64_t)(w.hi / (p.h / p.h_kv)) * p.k_sh;
    w.v_off = (int64_t)k0 * p.v_ss + (int64_t)(w.hi / (p.h / p.h_kv)) * p.v_sh;
    w.lse_off = (int64_t)q0 * p.h + w.hi;
    w.lse_st = p.h;
    pair = pu.j;
    n_qt = (w.q_len + kFwdBlockM - 1) / kFwdBlockM;
  } else {
    const int nbh = p.b * p.h;
    pair = unit / nbh;
    const int bh = unit % nbh;
    const int bi = bh / p.h;
    w.hi = bh % p.h;
    w.q_len = p.s_q;
    w.kv_len = p.s_kv;
    w.q_off = (int64_t)bi * p.q_sb + (int64_t)w.hi * p.q_sh;
    w.o_off = (int64_t)bi * p.o_sb + (int64_t)w.hi * p.o_sh;
    w.k_off = (int64_t)bi * p.k_sb + (int64_t)(w.hi / (p.h / p.h_kv)) * p.k_sh;
    w.v_off = (int64_t)bi * p.v_sb + (int64_t)(w.hi / (p.h / p.h_kv)) * p.v_sh;
    w.lse_off = ((int64_t)bi * p.h + w.hi) * p.s_q;
    w.lse_st = 1;
    n_qt = p.n_qtiles;
  }
  const int first = heavy ? n_qt - 1 - pair : 2 * pair;
  const int second0 = heavy ? pair : 2 * pair + 1;
  const int second = (heavy ? second0 < first : second0 < n_qt) ? second0 : -1;
  w.qt = half ? second : first;
  if (w.qt < 0) {
    w.qt = 0;
    w.q_len = 0;
  }
  return w;
}

// Per-lane softmax state update for one tile of 32 scores held in s[2][16]
// (already masked with -inf). Returns alpha, the factor for the old O.
__device__ __forceinline__ float softmax_tile(f32x16 (&s)[2], float c, float& m_run,
                                              float& l_run) {
  float mx = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
  mx = fmaxf(mx, other_half(mx));
  const float m_new = fmaxf(m_run, mx * c);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = fast_exp2(m_run - m_use);
  float rs = 0.f;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pv = fast_exp2(fmaf(s[mb][r], c, -m_use));
      s[mb][r] = pv;
      rs += pv;
    }
  l_run = l_run * alpha + rs;
  m_run = m_new;
  return alpha;
}

// Key index held by register r of block mb of S^T in a lane of half hf.
__device__ __forceinline__ int s_key(int mb, int r, int hf) {
  return 32 * mb + 8 * (r / 4) + 4 * hf + (r % 4);
}

// Masks every score of a tile (a neutralised softmax).
__device__ __forceinline__ void mask_all(f32x16 (&s)[2]) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[mb][r] = -INFINITY;
}

// Hides the scores of keys outside the band of each row of a tile: key >
// qi + shift (causal), key < qi + shift - window, key >= kv_len. shift = 0
// (top-left) or kv_len - q_len (bottom-right); window is a huge value when
// there is no left bound. Each bound is applied only when it cuts the tile
// (the caller's wave-uniform flags), as one compare per score of the key's
// offset in the tile (a constant per register, plus 4 hf) against a per-lane
// limit and a select (a conditional store instead became a chain of
// exec-mask updates).
template <bool CAUSAL>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], int kbase, int qi, int kv_len, int hf,
                                          int shift, int window, bool cut_causal, bool cut_left,
                                          bool cut_end) {
  const int base = kbase + 4 * hf;  // key of offset s_key(mb, r, 0) is base + that offset
  if (CAUSAL && cut_causal) {
    const int lim = qi + shift - base;  // visible iff offset <= lim
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mb][r] = s_key(mb, r, 0) > lim ? -INFINITY : s[mb][r];
  }
  if (cut_left) {
    const int lim = qi + shift - window - base;  // visible iff offset >= lim
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mb][r] = s_key(mb, r, 0) < lim ? -INFINITY : s[mb][r];
  }
  if (cut_end) {
    const int lim = kv_len - base;  // visible iff offset < lim
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mb][r] = s_key(mb, r, 0) >= lim ? -INFINITY : s[mb][r];
  }
}

}  // namespace
}  // namespace sdpa07
