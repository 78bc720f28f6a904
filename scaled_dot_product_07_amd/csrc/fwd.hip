// Fused scaled-dot-product attention forward for gfx950 (MI355X).
//
// Computes O = softmax(scale * Q K^T + mask) V and the natural-log row
// statistic LSE for dense (b, h, s, d) batches and packed THD batches
// ("Inside NVIDIA's cuDNN Graph API ...", section 5: the operation, scale and
// top-left causal band; cudnn-frontend PR #554: statistic layouts and THD
// packing with cu_seqlens).
//
// One workgroup = 4 waves = 128 query rows of one (b, h) or (sequence, h).
// Each wave owns 32 query rows and keeps, for the whole key loop:
//   * its Q rows as MFMA B operands in VGPRs (loaded once),
//   * the fp32 output accumulator O^T (d x 32) in the MFMA C layout,
//   * the running max m and running sum l of its rows.
// Keys are streamed in tiles of 64 rows of K and V through double-buffered
// LDS: the global loads of tile j+1 are issued before tile j is computed and
// written to the other buffer after it, with one barrier per tile.
//
// The products are computed transposed, S^T = K Q^T and O^T = V^T P^T, on
// v_mfma_f32_32x32x16_{bf16,f16} (v_mfma_f32_32x32x2_f32 for fp32 io). In
// the C layout of S^T a lane holds one query column and 16 key rows, so the
// row max and row sum of the softmax are in-lane reductions plus one swap
// between the two 32-lane halves (v_permlane32_swap). P^T leaves the
// accumulator already in the B-operand layout of the P.V product once the
// contraction index is relabelled (the relabelling is matched on the V side
// by the transposing LDS read ds_read_b64_tr_b16), so P never goes through
// LDS.
//
// Online softmax in base 2: c = |scale| * log2(e), m' = max(m, c * rowmax S),
// P = 2^(c*S - m'), alpha = 2^(m - m'), l' = alpha*l + rowsum P,
// O' = alpha*O + P V; at the end O = O / l and LSE = ln2 * (m + log2 l).
// A negative scale is moved onto Q as an exact sign flip so that c > 0.
//
// Causal (top-left): query i sees key j iff j <= i. Key tiles past the last
// visible key of the workgroup are never loaded; a wave skips the tiles past
// its own last visible key, and only tiles that straddle the diagonal (or the
// end of the keys) evaluate the mask. Loads of key rows at or beyond the
// sequence's key count are predicated off and zero-filled, so padding or a
// NaN-poisoned tail never reaches P.V (the FP8 d512 forward entry in the
// cudnn-frontend PR #554 merge log describes that failure: masking zeroes P,
// not V).
//
// Work order: blockIdx -> (query tile, b*h) with the heaviest causal query
// tiles first (longest-processing-time order), and all tiles of one (b, h)
// on the same XCD when b*h is a multiple of 8, so they share its L2.

#include <math.h>

#include <type_traits>

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

template <bool VARLEN>
__device__ __forceinline__ Unit decode_unit(const FwdParams& p) {
  Unit w;
  const int nbh = p.b * p.h;
  const int u = blockIdx.x;
  w.qt = p.n_qtiles - 1 - u / nbh;  // heaviest causal tiles first
  const int bh = u % nbh;
  const int bi = bh / p.h;
  w.hi = bh % p.h;
  if constexpr (VARLEN) {
    const int q0 = min(max(p.cu_q[bi], 0), p.total_q);
    const int q1 = min(max(p.cu_q[bi + 1], 0), p.total_q);
    const int k0 = min(max(p.cu_kv[bi], 0), p.total_kv);
    const int k1 = min(max(p.cu_kv[bi + 1], 0), p.total_kv);
    w.q_len = max(q1 - q0, 0);
    w.kv_len = max(k1 - k0, 0);
    w.q_off = (int64_t)q0 * p.q_ss + (int64_t)w.hi * p.q_sh;
    w.o_off = (int64_t)q0 * p.o_ss + (int64_t)w.hi * p.o_sh;
    w.k_off = (int64_t)k0 * p.k_ss + (int64_t)w.hi * p.k_sh;
    w.v_off = (int64_t)k0 * p.v_ss + (int64_t)w.hi * p.v_sh;
    w.lse_off = (int64_t)q0 * p.h + w.hi;
    w.lse_st = p.h;
  } else {
    w.q_len = p.s_q;
    w.kv_len = p.s_kv;
    w.q_off = (int64_t)bi * p.q_sb + (int64_t)w.hi * p.q_sh;
    w.o_off = (int64_t)bi * p.o_sb + (int64_t)w.hi * p.o_sh;
    w.k_off = (int64_t)bi * p.k_sb + (int64_t)w.hi * p.k_sh;
    w.v_off = (int64_t)bi * p.v_sb + (int64_t)w.hi * p.v_sh;
    w.lse_off = ((int64_t)bi * p.h + w.hi) * p.s_q;
    w.lse_st = 1;
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

template <bool CAUSAL>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], int kbase, int qi, int kv_len,
                                          int hf) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kbase + s_key(mb, r, hf);
      if ((CAUSAL && key > qi) || key >= kv_len) s[mb][r] = -INFINITY;
    }
}

// ---------------------------------------------------------------------------
// fp16 / bf16 io.
//
// A workgroup of 8 waves owns a PAIR of 128-row query tiles of one head: tile
// i (waves 0-3) and tile n-1-i (waves 4-7). Under the causal mask their key
// counts sum to the same total for every pair, so every workgroup (and every
// SIMD, which runs one wave of each tile) gets the same work; the key tiles
// the short tile needs are a prefix of the long tile's and are loaded once.
//
// Per wave and key tile the work is software-pipelined: the QK^T products of
// tile j+1 are issued in the same basic block as the softmax of tile j, so
// the exp/convert/max VALU work fills the MFMA pipeline's issue gaps; the
// P.V products of tile j then overlap the row sums. The running max used as
// the exponent offset is only raised when a tile's max exceeds it by more
// than kTau (log2 units), so P <= 2^kTau and the O accumulator is rescaled
// only on those (rare) tiles; the result is exact either way because O and l
// always share the same offset.
constexpr float kTau = 8.f;

template <typename T, int D, bool CAUSAL, bool VARLEN>
__global__ void __launch_bounds__(kFwdThreads16) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd16_kernel(FwdParams p) {
  constexpr int BM = kFwdBlockM, BN = kFwdBlockN;
  constexpr int NT = kFwdThreads16;
  constexpr int PITCH = D + 8;  // LDS row pitch (elements); +16 B breaks bank aliasing
  constexpr int CH_ROW = D / 8;  // 16-byte chunks per row
  constexpr int CPT = BN * CH_ROW / NT;  // chunks per thread per tensor per tile
  static_assert(CPT >= 1, "tile too small for the workgroup");
  using M = Mfma16<T>;
  using v8 = typename M::v8;
  __shared__ __attribute__((aligned(16))) T kl[2][BN * PITCH];
  __shared__ __attribute__((aligned(16))) T vl[2][BN * PITCH];

  // ---- work unit: (query tile, b|sequence, h). Query tiles are ordered as a
  // snake, heaviest causal tile first: n-1, n-2, .., n/2, then 0, 1, .., so the
  // two workgroups resident on a CU (dispatched nbh*ceil(n/2) apart) pair a
  // heavy tile with a light one.
  const int nbh = p.b * p.h;
  const int urow = blockIdx.x / nbh;
  const int bh = blockIdx.x % nbh;
  const int half = (p.n_qtiles + 1) / 2;
  const int qt_sched = urow < half ? p.n_qtiles - 1 - urow : urow - half;
  const int bi = bh / p.h, hi = bh % p.h;
  int q_len, kv_len;
  int64_t q_off, k_off, v_off, o_off, lse_off, lse_st;
  if constexpr (VARLEN) {
    const int q0 = min(max(p.cu_q[bi], 0), p.total_q);
    const int q1 = min(max(p.cu_q[bi + 1], 0), p.total_q);
    const int k0 = min(max(p.cu_kv[bi], 0), p.total_kv);
    const int k1 = min(max(p.cu_kv[bi + 1], 0), p.total_kv);
    q_len = max(q1 - q0, 0);
    kv_len = max(k1 - k0, 0);
    q_off = (int64_t)q0 * p.q_ss + (int64_t)hi * p.q_sh;
    o_off = (int64_t)q0 * p.o_ss + (int64_t)hi * p.o_sh;
    k_off = (int64_t)k0 * p.k_ss + (int64_t)hi * p.k_sh;
    v_off = (int64_t)k0 * p.v_ss + (int64_t)hi * p.v_sh;
    lse_off = (int64_t)q0 * p.h + hi;
    lse_st = p.h;
  } else {
    q_len = p.s_q;
    kv_len = p.s_kv;
    q_off = (int64_t)bi * p.q_sb + (int64_t)hi * p.q_sh;
    o_off = (int64_t)bi * p.o_sb + (int64_t)hi * p.o_sh;
    k_off = (int64_t)bi * p.k_sb + (int64_t)hi * p.k_sh;
    v_off = (int64_t)bi * p.v_sb + (int64_t)hi * p.v_sh;
    lse_off = ((int64_t)bi * p.h + hi) * p.s_q;
    lse_st = 1;
  }
  if (qt_sched * BM >= q_len) return;  // uniform over the workgroup, before any barrier

  const T* __restrict__ Q = (const T*)p.q + q_off;
  const T* __restrict__ K = (const T*)p.k + k_off;
  const T* __restrict__ V = (const T*)p.v + v_off;
  T* __restrict__ O = (T*)p.o + o_off;

  const int tid = threadIdx.x, lane = tid % 64;
  // wave-uniform values live in SGPRs so per-wave control flow stays scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int hf = lane / 32, col = lane % 32;
  const int qt = qt_sched;
  const int row0 = qt * BM + wave * 32;
  const int qi = row0 + col;
  const bool wave_active = row0 < q_len;
  const bool q_valid = wave_active && qi < q_len;
  const int last_q = min(q_len, (qt + 1) * BM) - 1;
  const int kv_end = CAUSAL ? min(kv_len, last_q + 1) : kv_len;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const int wave_kv_end =
      !wave_active ? 0 : (CAUSAL ? min(kv_len, min(q_len, row0 + 32)) : kv_len);
  const int wave_tiles = (wave_kv_end + BN - 1) / BN;

  v8 qf[D / 16];
  i16x8 qraw[D / 16];
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  float l_run = 0.f;
  const float c = p.scale_log2;

  // K/V tile loads through a buffer resource rebased per tile whose byte
  // bound ends with the last key row of the sequence: loads of rows past it
  // read as zeros (rows are disjoint when the row stride is at least d, which
  // every dense layout satisfies; with overlapping rows the extra rows are
  // real, finite keys that the mask hides), with no per-lane test and no
  // memory touched past the keys.
  int kroff[CPT], vroff[CPT];
#pragma unroll
  for (int x = 0; x < CPT; ++x) {
    const int ch = tid + NT * x;
    const int r = ch / CH_ROW, cc = ch % CH_ROW;
    kroff[x] = r * (int)p.k_ss * (int)sizeof(T) + cc * 16;
    vroff[x] = r * (int)p.v_ss * (int)sizeof(T) + cc * 16;
  }
  // K/V tiles are staged through registers PD tiles ahead of their LDS store
  // (two stages where registers allow), so global latency is covered by PD
  // pipeline steps
  constexpr int PD = D <= 64 ? 2 : 1;
  i16x8 kreg[PD][CPT], vreg[PD][CPT];
  auto gload = [&](i16x8(&reg)[CPT], const T* __restrict__ base, int64_t stride,
                   const int(&roff)[CPT], int j) {
    const T* tb = base + (int64_t)j * BN * stride;
    const int rows = min(kv_len - j * BN, BN);
    const int bytes = rows <= 0 ? 0 : ((rows - 1) * (int)stride + D) * (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)tb, (short)0, bytes, kBufferFlags);
#pragma unroll
    for (int x = 0; x < CPT; ++x)
      reg[x] = __builtin_bit_cast(i16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, roff[x], 0, 0));
  };
  auto lstore = [&](T* buf, const i16x8(&reg)[CPT]) {
#pragma unroll
    for (int x = 0; x < CPT; ++x) {
      const int ch = tid + NT * x;
      const int r = ch / CH_ROW, cc = ch % CH_ROW;
      *(i16x8*)&buf[r * PITCH + cc * 8] = reg[x];
    }
  };
  // Softmax state (per lane = per query row, both halves agree):
  //   m_cur  offset of P_j (log2 units) for the tile the next block exponentiates
  //   a_cur  2^(m_prev - m_cur): factor for l (in that block) and for O (after it)
  //   m_prev offset of the previous tile (kept to redo the update after a mask)
  //   m_l    offset of l (and of O once the pending P.V is added): the LSE base
  float m_prev = -INFINITY, m_cur = -INFINITY, a_cur = 0.f, m_l = -INFINITY;
  // lazy offset update from a tile max (raw score units): raise the offset
  // only when the tile's max exceeds it by more than kTau
  auto offset_update = [&](float mx, float m_from, float& m_to, float& a) {
    const float mt = mx * c;
    const float m_new = mt > m_from + kTau ? mt : m_from;
    a = fast_exp2(m_from - (m_new == -INFINITY ? 0.f : m_new));
    m_to = m_new;
  };
  auto row_max = [&](const f32x16(&sv)[2]) -> float {
    float a = fmaxf(sv[0][0], sv[0][1]), b = fmaxf(sv[1][0], sv[1][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) {
      a = fmaxf(a, fmaxf(sv[0][r], sv[0][r + 1]));
      b = fmaxf(b, fmaxf(sv[1][r], sv[1][r + 1]));
    }
    const float mx = fmaxf(a, b);
    return fmaxf(mx, other_half(mx));
  };

  // One pipeline block for key tile j of this wave, straight-line code:
  //   QK  : S_{j+1} = K_{j+1} Q^T                (MFMAs 0 .. NQK-1)
  //   PV  : O^T += V_{j-1}^T P_{j-1}^T             (MFMAs NQK .. NM-1)
  //   SM  : P_j = 2^(c S_j - m_cur), row sum into l (VALU, early chunks)
  //   MX  : row max of S_{j+1} and the next offset (VALU, last chunks, once
  //         the QK results are complete)
  // It is emitted as NM chunks, each = the LDS read for the MFMA PF chunks
  // ahead, one MFMA, and a slice of the VALU work; the slices are pinned to
  // their chunk so the VALU work issues while the MFMA pipe is busy.
  constexpr int NQK = 2 * (D / 16);
  constexpr int NPV = 4 * (D / 32);
  constexpr int NM = NQK + NPV;
  constexpr int PF = 3;                                   // LDS read-ahead (chunks)
  constexpr int NPAIR = 16;                               // 32 scores per lane, in pairs
  constexpr int EXP_CHUNKS = NM - 6 < 16 ? NM - 6 : 16;   // chunks holding the exps
  constexpr int MX0 = NM - 4;                             // chunks MX0 .. MX0+2: max of S_{j+1}
  const int vrow = 4 * hf + (lane % 16) / 4;
  const int vcol = 16 * ((lane / 16) % 2) + 4 * (lane % 4);
  auto block = [&](const T* kb, const T* vb, const f32x16(&s_cur)[2], f32x16(&s_nxt)[2],
                   const v8(&p_prev)[4], v8(&p_cur)[4]) {
    auto read_op = [&](int i) -> v8 {
      if (i < NQK) {
        const int ks = i / 2, mb = i % 2;
        return *(const v8*)&kb[(32 * mb + col) * PITCH + 16 * ks + 8 * hf];
      }
      const int t = (i - NQK) / (D / 32), db = (i - NQK) % (D / 32);
      const T* a0 = vb + (16 * t + vrow) * PITCH + 32 * db + vcol;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(a0));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(a0 + 8 * PITCH));
      return __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    const float m_off = m_cur == -INFINITY ? 0.f : m_cur;
    m_l = m_cur;
    float r0 = 0.f, r1 = 0.f, mxa = -INFINITY, mxb = -INFINITY;
    i32x4 pk[4];
    auto slice = [&](int i) {
      if (i < EXP_CHUNKS) {
        const int p0 = i * NPAIR / EXP_CHUNKS, p1 = (i + 1) * NPAIR / EXP_CHUNKS;
#pragma unroll
        for (int pp = p0; pp < p1; ++pp) {
          const int t = pp / 4, e2 = pp % 4;
          const f32x2 x = {fast_exp2(fmaf(s_cur[t / 2][8 * (t % 2) + 2 * e2], c, -m_off)),
                           fast_exp2(fmaf(s_cur[t / 2][8 * (t % 2) + 2 * e2 + 1], c, -m_off))};
          const auto h = __builtin_convertvector(x, typename Pack2<T>::type);
          int hb = __builtin_bit_cast(int, h);
          pin(hb);
          pk[t][e2] = hb;
          if (e2 & 1) r1 = dot2_ones<T>(h, r1);
          else r0 = dot2_ones<T>(h, r0);
        }
      }
      if (i == EXP_CHUNKS) {
        l_run = l_run * a_cur + (r0 + r1);
        pin(l_run);
      }
      if (i == MX0) {
        mxa = fmaxf(fmaxf(s_nxt[0][0], s_nxt[0][1]), fmaxf(s_nxt[0][2], s_nxt[0][3]));
        mxb = fmaxf(fmaxf(s_nxt[0][4], s_nxt[0][5]), fmaxf(s_nxt[0][6], s_nxt[0][7]));
#pragma unroll
        for (int r = 8; r < 16; r += 2) {
          mxa = fmaxf(mxa, s_nxt[0][r]);
          mxb = fmaxf(mxb, s_nxt[0][r + 1]);
        }
        pin(mxa);
        pin(mxb);
      }
      if (i == MX0 + 1) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          mxa = fmaxf(mxa, s_nxt[1][r]);
          mxb = fmaxf(mxb, s_nxt[1][r + 1]);
        }
        pin(mxa);
        pin(mxb);
      }
      if (i == MX0 + 2) {
        float mx = fmaxf(mxa, mxb);
        mx = fmaxf(mx, other_half(mx));
        m_prev = m_cur;
        offset_update(mx, m_cur, m_cur, a_cur);
        pin(m_cur);
        pin(a_cur);
      }
    };
    v8 op[NM];
#pragma unroll
    for (int i = 0; i < PF; ++i) op[i] = read_op(i);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i + PF < NM) op[i + PF] = read_op(i + PF);
      if (i < NQK) {
        const int ks = i / 2, mb = i % 2;
        s_nxt[mb] = M::mma(op[i], qf[ks], ks == 0 ? f32x16{} : s_nxt[mb]);
      } else {
        const int t = (i - NQK) / (D / 32), db = (i - NQK) % (D / 32);
        acc[db] = M::mma(op[i], p_prev[t], acc[db]);
      }
      slice(i);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) p_cur[t] = __builtin_bit_cast(v8, pk[t]);
  };

  // The per-tile step. Every pipeline block runs the same fused code; the
  // edges are neutralised by data instead of separate code paths: a zero
  // P_{j-1} (and a zeroed V buffer) makes PV a no-op, a fully masked S_j
  // makes the softmax a no-op (P = 0), and an unneeded QK only computes a
  // value that is never used. A wave skips the tiles past its causal range
  // (j > wave_tiles) except for the memory work the whole workgroup shares.
  // `par` is j mod 2, known at compile time (the loop is unrolled by two)
  auto step = [&](int j, auto par, f32x16(&s_cur)[2], f32x16(&s_nxt)[2],
                  const v8(&p_prev)[4], v8(&p_cur)[4]) {
    constexpr int J = decltype(par)::value;
    constexpr int KS = (J + 1) % PD, VS = J % PD;  // register stages of K_{j+1}, V_j
    // K_{j+1} into LDS (its global load was issued PD blocks ago); the loads
    // and stores run unconditionally so that wait counts stay exact (a load
    // past the keys reads zeros through the buffer bound)
    lstore(kl[(j + 1) & 1], kreg[KS]);
    __syncthreads();
    lstore(vl[j & 1], vreg[VS]);
    gload(vreg[VS], V, p.v_ss, vroff, j + PD);
    gload(kreg[KS], K, p.k_ss, kroff, j + 1 + PD);
    if (j <= wave_tiles) {
      const int kbase = j * BN;
      if (j == wave_tiles) {
        mask_all(s_cur);  // past this wave's range: a neutralised softmax
        m_cur = m_prev;
        a_cur = 1.f;
      } else if ((CAUSAL && kbase + BN - 1 > row0) || kbase + BN > kv_len) {
        mask_tile<CAUSAL>(s_cur, kbase, qi, kv_len, hf);
        offset_update(row_max(s_cur), m_prev, m_cur, a_cur);  // redo with the mask
      }
      const bool rescale = __any(a_cur != 1.f);
      const float a_blk = a_cur;
      block(kl[(j + 1) & 1], vl[(j - 1) & 1], s_cur, s_nxt, p_prev, p_cur);
      if (rescale) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] *= a_blk;
      }
    }
  };

  if (n_tiles > 0) {
    f32x16 sa[2], sb[2];
    v8 pa[4], pb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      pa[t] = v8{};
      pb[t] = v8{};
    }
    gload(kreg[0], K, p.k_ss, kroff, 0);
#pragma unroll
    for (int t = 0; t < PD; ++t) gload(vreg[t], V, p.v_ss, vroff, t);
    // Q rows as B operands of S^T = K Q^T (lane holds Q[qi][16ks + 8hf .. +7]),
    // loaded after the first K/V tiles are requested so that the two
    // latencies overlap; rows past the sequence read as zeros
    {
      const T* qb = Q + (int64_t)(qt * BM) * p.q_ss;
      const int rows = min(q_len - qt * BM, BM);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)qb, (short)0, ((rows - 1) * (int)p.q_ss + D) * (int)sizeof(T), kBufferFlags);
      const int qoff = (qi - qt * BM) * (int)p.q_ss * (int)sizeof(T) + 16 * hf;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        qraw[ks] = __builtin_bit_cast(i16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, qoff + 32 * ks, 0, 0));
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      i16x8 raw = qraw[ks];
      if (p.negate_q) raw ^= (short)0x8000;
      qf[ks] = __builtin_bit_cast(v8, raw);
    }
    lstore(kl[0], kreg[0]);
    {
      const i16x8 zero[CPT] = {};
      lstore(vl[1], zero);  // read by the no-op P.V of the first block
    }
#pragma unroll
    for (int t = 1; t <= PD; ++t) gload(kreg[t % PD], K, p.k_ss, kroff, t);
    __syncthreads();
    // S_0 = QK(K_0) and its offset; the P.V and softmax parts are neutralised
    // (sb fully masked, P_{-1} = 0, V buffer 1 zero)
    mask_all(sb);
    block(kl[0], vl[1], sb, sa, pb, pa);
    int j = 0;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    for (; j + 1 < n_tiles; j += 2) {
      step(j, I0{}, sa, sb, pb, pa);
      step(j + 1, I1{}, sb, sa, pa, pb);
    }
    if (j < n_tiles) {
      step(j, I0{}, sa, sb, pb, pa);
      ++j;
    }
    // drain: P.V of the last tile, whose V was stored in the last block; the
    // block's softmax is neutralised (masked scores, factor 1 at the offset
    // of l), and its new offset comes from unused scores and is discarded
    __syncthreads();
    if (j - 1 < wave_tiles) {
      m_cur = m_l;
      a_cur = 1.f;
      if ((j - 1) & 1) {
        mask_all(sa);
        block(kl[0], vl[1], sa, sb, pb, pa);
      } else {
        mask_all(sb);
        block(kl[0], vl[0], sb, sa, pa, pb);
      }
    }
  }

  // Epilogue: combine the two halves' partial sums, normalise, store.
  const float l_tot = l_run + other_half(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_valid) {
    T* orow = O + (int64_t)qi * p.o_ss;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        typedef T t4 __attribute__((ext_vector_type(4)));
        t4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (T)(acc[db][4 * rq + e] * inv);
        *(t4*)(orow + 32 * db + 8 * rq + 4 * hf) = ov;
      }
    if (hf == 0 && p.lse)
      p.lse[lse_off + (int64_t)qi * lse_st] =
          l_tot > 0.f ? (m_l + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// fp32 io: the same schedule on v_mfma_f32_32x32x2_f32 (full fp32 products).
// With one k element per lane no transposed read is needed: the PV product
// takes V rows directly from LDS, P straight from the S^T accumulator.
template <int D, bool CAUSAL, bool VARLEN>
__global__ void __launch_bounds__(kFwdThreads) fwd32_kernel(FwdParams p) {
  constexpr int BM = kFwdBlockM, BN = kFwdBlockN;
  constexpr int PITCH = D + 4;
  constexpr int CH_ROW = D / 4;
  constexpr int CPT = BN * CH_ROW / kFwdThreads;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) float lds[2][2][BN * PITCH];

  const Unit w = decode_unit<VARLEN>(p);
  if (w.qt * BM >= w.q_len) return;

  const float* __restrict__ Q = (const float*)p.q + w.q_off;
  const float* __restrict__ K = (const float*)p.k + w.k_off;
  const float* __restrict__ V = (const float*)p.v + w.v_off;
  float* __restrict__ O = (float*)p.o + w.o_off;

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int hf = lane / 32, col = lane % 32;
  const int row0 = w.qt * BM + wave * 32;
  const int qi = row0 + col;
  const bool q_valid = qi < w.q_len;
  const bool wave_active = row0 < w.q_len;
  const int blk_last_q = min(w.q_len, (w.qt + 1) * BM) - 1;
  const int kv_end = CAUSAL ? min(w.kv_len, blk_last_q + 1) : w.kv_len;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const int wave_kv_end = CAUSAL ? min(w.kv_len, min(w.q_len, row0 + 32)) : w.kv_len;

  float qf[D / 2];
#pragma unroll
  for (int ks = 0; ks < D / 2; ++ks) {
    float x = q_valid ? Q[(int64_t)qi * p.q_ss + 2 * ks + hf] : 0.f;
    qf[ks] = p.negate_q ? -x : x;
  }
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.scale_log2;

  f32x4 kreg[CPT], vreg[CPT];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int x = 0; x < CPT; ++x) {
      const int ch = tid + kFwdThreads * x;
      const int r = ch / CH_ROW, cc = ch % CH_ROW;
      const int key = j * BN + r;
      if (key < w.kv_len) {
        kreg[x] = *(const f32x4*)(K + (int64_t)key * p.k_ss + cc * 4);
        vreg[x] = *(const f32x4*)(V + (int64_t)key * p.v_ss + cc * 4);
      } else {
        kreg[x] = f32x4{};
        vreg[x] = f32x4{};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int x = 0; x < CPT; ++x) {
      const int ch = tid + kFwdThreads * x;
      const int r = ch / CH_ROW, cc = ch % CH_ROW;
      *(f32x4*)&lds[buf][0][r * PITCH + cc * 4] = kreg[x];
      *(f32x4*)&lds[buf][1][r * PITCH + cc * 4] = vreg[x];
    }
  };

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_tiles) load_tile(j + 1);
    const int kbase = j * BN;
    if (wave_active && kbase < wave_kv_end) {
      f32x16 s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < D / 2; ++ks) {
          const float a = lds[buf][0][(32 * mb + col) * PITCH + 2 * ks + hf];
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qf[ks], s[mb], 0, 0, 0);
        }
      }
      if ((CAUSAL && kbase + BN - 1 > row0) || kbase + BN > w.kv_len)
        mask_tile<CAUSAL>(s, kbase, qi, w.kv_len, hf);
      const float alpha = softmax_tile(s, c, m_run, l_run);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
      // O^T += V^T P^T, one key pair (k = hf) per MFMA.
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float a = lds[buf][1][s_key(mb, r, hf) * PITCH + 32 * db + col];
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[mb][r], acc[db], 0, 0, 0);
          }
    }
    if (j + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + other_half(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_valid) {
    float* orow = O + (int64_t)qi * p.o_ss;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        f32x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = acc[db][4 * rq + e] * inv;
        *(f32x4*)(orow + 32 * db + 8 * rq + 4 * hf) = ov;
      }
    if (hf == 0 && p.lse)
      p.lse[w.lse_off + (int64_t)qi * w.lse_st] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL, bool VARLEN>
const void* pick_kernel(Dt dt) {
  // fp16/bf16 kernels run 8-wave workgroups over pairs of query tiles;
  // the fp32 kernel runs 4-wave workgroups over single query tiles.
  switch (dt) {
    case Dt::BF16: return (const void*)&fwd16_kernel<__bf16, D, CAUSAL, VARLEN>;
    case Dt::F16: return (const void*)&fwd16_kernel<_Float16, D, CAUSAL, VARLEN>;
    case Dt::F32: return (const void*)&fwd32_kernel<D, CAUSAL, VARLEN>;
  }
  return nullptr;
}

template <int D>
const void* pick_kernel(Dt dt, bool causal, bool varlen) {
  if (causal) return varlen ? pick_kernel<D, true, true>(dt) : pick_kernel<D, true, false>(dt);
  return varlen ? pick_kernel<D, false, true>(dt) : pick_kernel<D, false, false>(dt);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, Dt dt, int d, bool causal, bool varlen,
                      hipStream_t stream) {
  const void* fn = d == 64 ? pick_kernel<64>(dt, causal, varlen)
                           : pick_kernel<128>(dt, causal, varlen);
  if (!fn) return hipErrorInvalidValue;
  const bool paired = dt != Dt::F32;
  const long long grid = (long long)p.n_qtiles * p.b * p.h;
  if (grid <= 0) return hipSuccess;
  FwdParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(paired ? kFwdThreads16 : kFwdThreads),
                         args, 0, stream);
}

}  // namespace sdpa07
