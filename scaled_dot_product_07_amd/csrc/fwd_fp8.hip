// FP8 (e4m3) scaled-dot-product attention forward for gfx950 (MI355X).
//
// Q, K, V hold e4m3 codes (OCP FP8, the format the gfx950 matrix cores and
// conversions use) with per-tensor factors: the real operands are
// descale_q * Q, descale_k * K, descale_v * V, and the output is stored as
// scale_o * O in bf16 or fp16, with the optional amax of the stored values
// before the cast. The factors are device scalars read by the kernel (no
// host readback); descale_q * descale_k folds into the log2 factor of the
// softmax, descale_v * scale_o into the epilogue's normalisation, and P is
// cast to e4m3 before the P.V product (cudnn-frontend PR #554 merge log, the
// per-tensor FP8 d512 forward entry; the FP8 forward of the same log casts P
// before BMM2). Masks, grouped-query heads and packed THD batches are those
// of the fp16/bf16 forward.
//
// One workgroup = 4 waves = one 128-row query tile of one (b, h) or
// (sequence, h); each wave owns 32 query rows. Keys are streamed in tiles of
// 64 rows of K and V through double-buffered LDS, filled by direct-to-LDS
// buffer loads of the next tile while the current one is computed. Both products run on
// v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3, fp32 accumulation), transposed as
// in the fp16/bf16 kernel:
//   S^T = K Q^T   A = 32 key rows x 64 d (two 16-byte LDS reads per lane),
//                 B = the wave's Q rows, kept in VGPRs;
//   O^T = V^T P^T B = P^T straight from the S^T accumulator: a lane holds the
//                 32 scores of one query whose keys k satisfy (k / 4) % 2 ==
//                 lane / 32, which is exactly one 64-deep B operand once the
//                 contraction slots are relabelled (slot 16b + 4q + i of half
//                 h = key 32b + 8q + 4h + i); A = V^T through the transposing
//                 byte read ds_read_b64_tr_b8 (lane i of a 16-lane group
//                 receives byte i % 8 of the 8-byte rows addressed by lanes
//                 2e + i / 8, e = 0..7), each lane addressing the V row its
//                 partner's slot needs;
//   sum           one more MFMA with a constant A whose row 0 is all ones
//                 gives the row sums of the rounded P in row 0 of its
//                 accumulator, so l is the exact fp32 sum of the P values the
//                 P.V product consumed.
// Online softmax in base 2 with a lazy offset: the offset m of a row rises
// only when a tile's max exceeds it by more than 4 (log2 units), and P is
// lifted by 2^4, so the row's largest P lies in [16, 256]: it always fits
// e4m3 (max 448), keeps 10 binades of smaller values in the normal range,
// and the accumulator rescale stays rare.

#include <limits.h>
#include <math.h>

#include "fwd_common.h"
#include "kernel_common.h"
#include "sdpa_internal.h"

namespace sdpa07 {
namespace {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kF8Threads = 256;
// P = 2^(c S - m + kF8Lift) with the offset m raised only when a tile's max
// exceeds it by more than kF8Tau: the largest P of a row lies in
// [2^kF8Lift, 2^(kF8Tau + kF8Lift)] = [16, 256], inside e4m3's finite range
// (448), and values down to 2^-10 of the row max stay normal (>= 2^-6)
constexpr float kF8Tau = 4.f;
constexpr float kF8Lift = 4.f;
constexpr int kE4M3One4 = 0x38383838;       // four e4m3 codes of 1.0
constexpr float kLog2eF = 1.4426950408889634f;

// e4m3 x e4m3 -> fp32, 32x32 output, 64-deep contraction (format codes 0, 0;
// zero scale operands select the unscaled instruction)
__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x2 read_tr8(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2*)(p));
}

// Four e4m3 codes of (a, b, c, d), round to nearest even.
__device__ __forceinline__ int pack4_e4m3(float a, float b, float c, float d) {
  int x = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, x, true);
}

template <typename TO>
struct Out4 {
  typedef TO type __attribute__((ext_vector_type(4)));
};

__global__ void zero_float_kernel(float* x) { *x = 0.f; }

template <typename TO, int D, bool CAUSAL, bool VARLEN>
__global__ void __launch_bounds__(kF8Threads) __attribute__((amdgpu_waves_per_eu(2)))
fwd8_kernel(FwdParams p) {
  constexpr int BM = kFwdBlockM, BN = kFwdBlockN;
  constexpr int CH = D / 16;                      // 16-byte chunks per row
  // K and V tiles in LDS: rows of D bytes, unpadded, whose 16-byte chunks
  // are permuted by an XOR of the row index (only r mod 16 matters; logical
  // chunk c of row r sits at c ^ swz(r)), so that the K reads (16 rows x one
  // chunk per ds_read_b128 phase), the V reads (rows {0..3, 8..11} + 4hf x
  // two chunks per 32-lane ds_read_b64_tr_b8 phase) and the tile stores all
  // hit distinct banks. No row padding serves the V reads: rows r and r + 8
  // of a phase would always share banks.
  auto swz = [](int r) -> int {
    if constexpr (D <= 64) {
      return (r >> 2) & 3;
    } else {
      const int k = (r >> 1) & 7;
      return 4 * (k & 1) + 2 * ((k >> 2) & 1) + ((k >> 1) & 1);
    }
  };
  // K and V tiles go from memory straight into LDS (buffer loads with the
  // LDS flag): a wave's load instruction fills 1 KB = RPI rows, lane l row
  // RIT(x) + l / CH, slot l % CH, with the global chunk that the slot holds
  // under the row's permutation; rows past the keys read as zeros (the
  // descriptor's byte bound ends with the last key row)
  constexpr int RPI = 1024 / D;                   // rows per load instruction
  constexpr int NW = kF8Threads / 64;             // waves
  constexpr int CPT = BN / (RPI * NW);            // load instructions per wave per tensor
  static_assert(CPT >= 1 && BN % (RPI * NW) == 0, "tile does not split over the waves");
  static_assert((NW * RPI) % 16 == 0, "load rows change the permutation phase");
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][2][BN * D];

  const Unit w = decode_unit_paired<VARLEN, CAUSAL>(p);
  if (w.qt * BM >= w.q_len) return;
  const unsigned char* __restrict__ Q = (const unsigned char*)p.q + w.q_off;
  const unsigned char* __restrict__ K = (const unsigned char*)p.k + w.k_off;
  const unsigned char* __restrict__ V = (const unsigned char*)p.v + w.v_off;
  TO* __restrict__ O = (TO*)p.o + w.o_off;

  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int hf = lane / 32, col = lane % 32;
  const int row0 = w.qt * BM + wave * 32;
  const int qi = row0 + col;
  const bool q_valid = qi < w.q_len;
  const bool wave_active = row0 < w.q_len;
  const int blk_last_q = min(w.q_len, (w.qt + 1) * BM) - 1;
  // band of row i: keys [i + shift - window, i + shift] (the upper bound only
  // when causal) within [0, kv_len); tiles [j0, j1) cover the workgroup's rows
  const int shift = p.bottom_right ? w.kv_len - w.q_len : 0;
  const int window = p.window_left < 0 ? (1 << 29) : p.window_left;
  const int kv_end = CAUSAL ? min(w.kv_len, max(blk_last_q + shift + 1, 0)) : w.kv_len;
  const int kv_begin = min(kv_end, max(w.qt * BM + shift - window, 0));
  const int j0 = kv_begin / BN, j1 = kv_end > kv_begin ? (kv_end + BN - 1) / BN : j0;
  const int wave_last = min(row0 + 31, w.q_len - 1);
  const int wave_kv_end = CAUSAL ? min(w.kv_len, max(wave_last + shift + 1, 0)) : w.kv_len;
  const int wave_kv_begin = max(row0 + shift - window, 0);

  // per-tensor factors: the effective score scale and the output factor
  const float dq = p.descale_q ? *p.descale_q : 1.f;
  const float dk = p.descale_k ? *p.descale_k : 1.f;
  const float dv = p.descale_v ? *p.descale_v : 1.f;
  const float so = p.scale_o ? *p.scale_o : 1.f;
  const float eff = p.scale * dq * dk;
  // |eff| * log2 e, kept > 0 so that -inf masks stay -inf; a negative
  // factor is moved onto Q as a sign flip (exact on e4m3 codes)
  const float c = fmaxf(fabsf(eff) * kLog2eF, 1e-30f);
  const int qsign = eff < 0.f ? (int)0x80808080 : 0;
  const float ofac = dv * so;

  // Q rows as B operands: lane holds Q[qi][64 kk + 32 hf .. + 31]
  i32x8 qf[D / 64];
#pragma unroll
  for (int kk = 0; kk < D / 64; ++kk) {
    i32x4 lo = {}, hi = {};
    if (q_valid) {
      const unsigned char* qp = Q + (int64_t)qi * p.q_ss + 64 * kk + 32 * hf;
      lo = *(const i32x4*)qp;
      hi = *(const i32x4*)(qp + 16);
    }
    qf[kk] = i32x8{lo[0] ^ qsign, lo[1] ^ qsign, lo[2] ^ qsign, lo[3] ^ qsign,
                   hi[0] ^ qsign, hi[1] ^ qsign, hi[2] ^ qsign, hi[3] ^ qsign};
  }
  // A operand of the row-sum product: row 0 all ones (lanes 0 and 32)
  const i32x8 ones = col == 0 ? i32x8{kE4M3One4, kE4M3One4, kE4M3One4, kE4M3One4, kE4M3One4,
                                      kE4M3One4, kE4M3One4, kE4M3One4}
                              : i32x8{};
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  f32x16 lacc = f32x16{};
  float m_off = -INFINITY;

  // V^T operand addressing: for transposing read j of d-block db, lane m
  // addresses the row of key 32(j/2) + 16(j%2) + 8(e/4) + 4h + e%4 (e =
  // (m % 16) / 2, h = m / 32) at byte 32 db + 16 ((m / 16) % 2) + 8 (m % 2)
  const int te = (lane % 16) / 2;
  const int v_row = 8 * (te / 4) + 4 * hf + te % 4;
  const int v_lane_off = v_row * D + 8 * (lane % 2);
  const int v_chunk = (lane / 16) % 2, v_swz = swz(v_row);
  const int k_swz = swz(col);  // rows 32mb + col

  auto RIT = [&](int x) { return (NW * x + wave) * RPI; };
  const int drow = lane / CH;
  const int dch = (lane % CH) ^ swz((RIT(0) + drow) % 16);  // RIT(x) mod 16: same for all x
  const int kvoff = drow * (int)p.k_ss + dch * 16;
  const int vvoff = drow * (int)p.v_ss + dch * 16;
  auto tile_rsrc = [&](const unsigned char* base, int64_t stride, int j) -> i32x4 {
    const int rows = min(w.kv_len - j * BN, BN);
    const int bytes = rows <= 0 ? 0 : (rows - 1) * (int)stride + D;
    const unsigned long long a = (unsigned long long)(base + (int64_t)j * BN * stride);
    return i32x4{(int)(unsigned)a, (int)((unsigned)(a >> 32) & 0xffffu), bytes, kBufferFlags};
  };
  auto lds_addr = [](const unsigned char* x) {
    return (unsigned)(size_t)(__attribute__((address_space(3))) const unsigned char*)x;
  };
  auto load_tile = [&](int j, int buf) {
    const i32x4 rk = tile_rsrc(K, p.k_ss, j), rv = tile_rsrc(V, p.v_ss, j);
#pragma unroll
    for (int x = 0; x < CPT; ++x)
      lds_dma16(rk, kvoff, RIT(x) * (int)p.k_ss, lds_addr(lds[buf][0] + RIT(x) * D));
#pragma unroll
    for (int x = 0; x < CPT; ++x)
      lds_dma16(rv, vvoff, RIT(x) * (int)p.v_ss, lds_addr(lds[buf][1] + RIT(x) * D));
  };

  if (j1 > j0) load_tile(j0, 0);
  // the Q rows above and the first tile have landed in every wave
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int j = j0; j < j1; ++j) {
    const int buf = (j - j0) & 1;
    if (j + 1 < j1) load_tile(j + 1, buf ^ 1);  // every wave is done with buf ^ 1
    const int kbase = j * BN;
    if (wave_active && kbase < wave_kv_end && kbase + BN > wave_kv_begin) {
      const unsigned char* kl = lds[buf][0];
      const unsigned char* vl = lds[buf][1];
      // S^T = K Q^T
      f32x16 s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 64; ++kk) {
          const unsigned char* kr = kl + (32 * mb + col) * D;
          const int c0 = 4 * kk + 2 * hf;  // logical chunks c0, c0 + 1
          const i32x4 lo = *(const i32x4*)(kr + ((c0 ^ k_swz) << 4));
          const i32x4 hi = *(const i32x4*)(kr + (((c0 + 1) ^ k_swz) << 4));
          const i32x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          s[mb] = mfma8(a, qf[kk], s[mb]);
        }
      }
      const bool cut_causal = CAUSAL && kbase + BN - 1 > row0 + shift;
      const bool cut_left = kbase < wave_last + shift - window;
      const bool cut_end = kbase + BN > w.kv_len;
      if (cut_causal || cut_left || cut_end)
        mask_tile<CAUSAL>(s, kbase, qi, w.kv_len, hf, shift, window, cut_causal, cut_left,
                          cut_end);
      // lazy offset: raise it (and rescale O and l) only when the tile's max
      // exceeds it by more than kF8Tau (the rescale factor is the same with
      // or without the lift)
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
      mx = fmaxf(mx, other_half(mx)) * c;
      const bool need = mx > m_off + kF8Tau;
      if (__any(need)) {
        const float m_new = need ? mx : m_off;
        const float alpha = need ? fast_exp2(m_off - m_new) : 1.f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
        lacc[0] *= alpha;
        m_off = m_new;
      }
      const float m_use = m_off == -INFINITY ? 0.f : m_off - kF8Lift;
      // P^T as the B operand: slot 16b + 4q + i of half h = key 32b + 8q + 4h + i
      i32x8 pb;
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        const int b = wd / 4, q4 = 4 * (wd % 4);
        pb[wd] = pack4_e4m3(fast_exp2(fmaf(s[b][q4], c, -m_use)),
                            fast_exp2(fmaf(s[b][q4 + 1], c, -m_use)),
                            fast_exp2(fmaf(s[b][q4 + 2], c, -m_use)),
                            fast_exp2(fmaf(s[b][q4 + 3], c, -m_use)));
      }
      // O^T += V^T P^T; l += rowsum(P) (row 0 of the ones product)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        // rows v_row + 16i keep v_row's permutation
        const unsigned char* vp = vl + v_lane_off + (((2 * db + v_chunk) ^ v_swz) << 4);
        const i32x2 r0 = read_tr8(vp);
        const i32x2 r1 = read_tr8(vp + 16 * D);
        const i32x2 r2 = read_tr8(vp + 32 * D);
        const i32x2 r3 = read_tr8(vp + 48 * D);
        const i32x8 a = {r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
        acc[db] = mfma8(a, pb, acc[db]);
      }
      lacc = mfma8(ones, pb, lacc);
    }
    // this wave's loads of tile j + 1 have landed; after the barrier every
    // wave's have, and every wave is done with buffer buf
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // l of this lane's query sits in row 0 of the ones product (half 0, reg 0)
  const float l_half = hf == 0 ? lacc[0] : 0.f;
  const float l_tot = l_half + other_half(l_half);
  const float inv = l_tot > 0.f ? ofac / l_tot : 0.f;
  float amax = 0.f;
  // The rows leave through LDS (free after the loop's last barrier): each
  // lane writes its 4-column pieces into the wave's 32 rows, laid out
  // [row][d] with the 16-byte chunks XOR-permuted by the row, then reads
  // back whole chunks, so that each store instruction writes complete rows
  // (with the system-scope cache policy, written through as stored); the
  // descriptor's byte bound drops the rows past the sequence.
  static_assert(NW * 32 * D * (int)sizeof(TO) <= (int)sizeof(lds), "staging rows exceed the LDS");
  TO* const stg = (TO*)&lds[0][0][0] + wave * 32 * D;
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int RPS = 64 / CPR;  // rows per store instruction
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      typename Out4<TO>::type ov;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = acc[db][4 * rq + e] * inv;
        if (q_valid) amax = fmaxf(amax, fabsf(x));
        ov[e] = (TO)x;
      }
      *(typename Out4<TO>::type*)&stg[col * D + ((4 * db + rq) ^ (col % CPR)) * 8 + 4 * hf] = ov;
    }
  // the wave reads back what its other lanes wrote (LDS operations of one
  // wave complete in order; the fences keep the compiler's order and wait)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  {
    const int sr = lane / CPR, sc = lane % CPR;
    i32x4 vrow[32 / RPS];
#pragma unroll
    for (int x = 0; x < 32 / RPS; ++x) {
      const int r = x * RPS + sr;
      vrow[x] = *(const i32x4*)&stg[r * D + (sc ^ (r % CPR)) * 8];
    }
    const int rows = wave_active ? min(w.q_len - row0, 32) : 0;
    if (p.o_ss < (1 << 24)) {
      const TO* base = O + (int64_t)max(row0, 0) * p.o_ss;
      const int bytes = rows <= 0 ? 0 : ((rows - 1) * (int)p.o_ss + D) * (int)sizeof(TO);
      const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, kBufferFlags);
      const int voff = (sr * (int)p.o_ss + sc * 8) * (int)sizeof(TO);
#pragma unroll
      for (int x = 0; x < 32 / RPS; ++x)
        __builtin_amdgcn_raw_buffer_store_b128(vrow[x], rs, voff,
                                               x * RPS * (int)p.o_ss * (int)sizeof(TO),
                                               kCacheSystemScope);
    } else {
#pragma unroll
      for (int x = 0; x < 32 / RPS; ++x) {
        const int r = x * RPS + sr;
        if (r < rows) *(i32x4*)(O + (int64_t)(row0 + r) * p.o_ss + sc * 8) = vrow[x];
      }
    }
  }
  if (q_valid) {
    if (hf == 0 && p.lse)
      p.lse[w.lse_off + (int64_t)qi * w.lse_st] =
          l_tot > 0.f ? (m_off - kF8Lift + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
  if (p.amax_o) {
    // non-negative floats order like their bit patterns
#pragma unroll
    for (int off = 32; off >= 1; off /= 2) amax = fmaxf(amax, __shfl_xor(amax, off));
    if (lane == 0) atomicMax((int*)p.amax_o, __builtin_bit_cast(int, amax));
  }
}

template <typename TO, int D>
const void* pick8(bool causal, bool varlen) {
  if (causal)
    return varlen ? (const void*)&fwd8_kernel<TO, D, true, true>
                  : (const void*)&fwd8_kernel<TO, D, true, false>;
  return varlen ? (const void*)&fwd8_kernel<TO, D, false, true>
                : (const void*)&fwd8_kernel<TO, D, false, false>;
}

}  // namespace

hipError_t launch_fwd_fp8(const FwdParams& p, Dt out, int d, bool causal, bool varlen,
                          hipStream_t stream) {
  const void* fn = nullptr;
  if (out == Dt::BF16)
    fn = d == 64 ? pick8<__bf16, 64>(causal, varlen) : pick8<__bf16, 128>(causal, varlen);
  else if (out == Dt::F16)
    fn = d == 64 ? pick8<_Float16, 64>(causal, varlen) : pick8<_Float16, 128>(causal, varlen);
  if (!fn) return hipErrorInvalidValue;
  if (p.amax_o) {
    float* a = p.amax_o;
    void* za[] = {&a};
    const hipError_t e =
        hipLaunchKernel((const void*)&zero_float_kernel, dim3(1), dim3(1), za, 0, stream);
    if (e != hipSuccess) return e;
  }
  // pairs of query tiles, one workgroup per tile (see decode_unit_paired)
  const long long units = varlen ? packed_units_per_head(p.total_q, p.b, 2 * kFwdBlockM) * p.h
                                 : (long long)((p.n_qtiles + 1) / 2) * p.b * p.h;
  if (units <= 0) return hipSuccess;
  const long long grid = 2 * units;
  if (grid > INT_MAX) return hipErrorInvalidValue;
  FwdParams arg = p;
  arg.split_round = compute_units();
  if (arg.split_round <= 0) return hipErrorInvalidDevice;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kF8Threads), args, 0, stream);
}

}  // namespace sdpa07
