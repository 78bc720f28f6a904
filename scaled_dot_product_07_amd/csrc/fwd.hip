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

#include "sdpa_internal.h"

namespace sdpa07 {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLn2 = 0.693147180559945309f;

template <typename T>
struct Mfma16;
template <>
struct Mfma16<__bf16> {
  using v8 = bf16x8;
  static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mfma16<_Float16> {
  using v8 = f16x8;
  static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// Value of x held by the lane 32 positions away (the other half-wave).
__device__ __forceinline__ float other_half(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  // Lanes < 32 receive the upper half in sw[1]; lanes >= 32 the lower in sw[0].
  const unsigned o = (threadIdx.x & 32) ? sw[0] : sw[1];
  return __builtin_bit_cast(float, o);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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
template <typename T, int D, bool CAUSAL, bool VARLEN>
__global__ void __launch_bounds__(kFwdThreads) fwd16_kernel(FwdParams p) {
  constexpr int BM = kFwdBlockM, BN = kFwdBlockN;
  constexpr int PITCH = D + 8;  // LDS row pitch (elements); +16 B breaks bank aliasing
  constexpr int CH_ROW = D / 8;  // 16-byte chunks per row
  constexpr int CPT = BN * CH_ROW / kFwdThreads;  // chunks per thread per tensor
  using M = Mfma16<T>;
  using v8 = typename M::v8;
  __shared__ __attribute__((aligned(16))) T lds[2][2][BN * PITCH];

  const Unit w = decode_unit<VARLEN>(p);
  if (w.qt * BM >= w.q_len) return;  // uniform over the workgroup, before any barrier

  const T* __restrict__ Q = (const T*)p.q + w.q_off;
  const T* __restrict__ K = (const T*)p.k + w.k_off;
  const T* __restrict__ V = (const T*)p.v + w.v_off;
  T* __restrict__ O = (T*)p.o + w.o_off;

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int hf = lane / 32, col = lane % 32;
  const int row0 = w.qt * BM + wave * 32;  // first query row of this wave
  const int qi = row0 + col;               // this lane's query row
  const bool q_valid = qi < w.q_len;
  const bool wave_active = row0 < w.q_len;
  const int blk_last_q = min(w.q_len, (w.qt + 1) * BM) - 1;
  const int kv_end = CAUSAL ? min(w.kv_len, blk_last_q + 1) : w.kv_len;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const int wave_kv_end = CAUSAL ? min(w.kv_len, min(w.q_len, row0 + 32)) : w.kv_len;

  // Q rows as B operands of S^T = K Q^T: lane holds Q[qi][16ks + 8hf .. +7].
  v8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    i16x8 raw = {};
    if (q_valid) raw = *(const i16x8*)(Q + (int64_t)qi * p.q_ss + 16 * ks + 8 * hf);
    if (p.negate_q) raw ^= (short)0x8000;
    qf[ks] = __builtin_bit_cast(v8, raw);
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.scale_log2;

  i16x8 kreg[CPT], vreg[CPT];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int x = 0; x < CPT; ++x) {
      const int ch = tid + kFwdThreads * x;
      const int r = ch / CH_ROW, cc = ch % CH_ROW;
      const int key = j * BN + r;
      if (key < w.kv_len) {
        kreg[x] = *(const i16x8*)(K + (int64_t)key * p.k_ss + cc * 8);
        vreg[x] = *(const i16x8*)(V + (int64_t)key * p.v_ss + cc * 8);
      } else {
        kreg[x] = i16x8{};
        vreg[x] = i16x8{};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int x = 0; x < CPT; ++x) {
      const int ch = tid + kFwdThreads * x;
      const int r = ch / CH_ROW, cc = ch % CH_ROW;
      *(i16x8*)&lds[buf][0][r * PITCH + cc * 8] = kreg[x];
      *(i16x8*)&lds[buf][1][r * PITCH + cc * 8] = vreg[x];
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
      // S^T (64 keys x 32 queries) = K_tile Q^T.
      f32x16 s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const v8 a = *(const v8*)&lds[buf][0][(32 * mb + col) * PITCH + 16 * ks + 8 * hf];
          s[mb] = M::mma(a, qf[ks], s[mb]);
        }
      }
      if ((CAUSAL && kbase + BN - 1 > row0) || kbase + BN > w.kv_len)
        mask_tile<CAUSAL>(s, kbase, qi, w.kv_len, hf);
      const float alpha = softmax_tile(s, c, m_run, l_run);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;

      // P^T as B operands: MFMA t covers keys 16t + 8(e/4) + 4hf + e%4.
      v8 pf[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[t][e] = (T)s[t / 2][8 * (t % 2) + e];

      // O^T += V^T P^T. The transposing LDS read gives lane (16-group g,
      // index i) V[kb + 0..3][dcol + i] with kb = 16t + 4hf, which is the
      // A operand for the same key relabelling.
      const T* vb = &lds[buf][1][0];
      const int vrow = 4 * hf + (lane % 16) / 4;
      const int vcol = 16 * ((lane / 16) % 2) + 4 * (lane % 4);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const T* a0 = vb + (16 * t + vrow) * PITCH + 32 * db + vcol;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(a0));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(a0 + 8 * PITCH));
          const i16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          acc[db] = M::mma(__builtin_bit_cast(v8, a), pf[t], acc[db]);
        }
    }
    if (j + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
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
      p.lse[w.lse_off + (int64_t)qi * w.lse_st] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
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
  const long long grid = (long long)p.n_qtiles * p.b * p.h;
  if (grid <= 0) return hipSuccess;
  FwdParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kFwdThreads), args, 0, stream);
}

}  // namespace sdpa07
