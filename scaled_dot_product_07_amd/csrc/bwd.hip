// Scaled-dot-product attention backward for gfx950 (MI355X).
//
// Given Q, K, V, O, dO and the forward's row statistic LSE, computes
//   P = exp(scale * Q K^T - LSE)  (the forward's softmax, recomputed),
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q
// (cudnn-frontend PR #554: the dense backward returns dQ, dK, dV from Q, K, V,
// O, dO and the statistic; its merge log, the SM80 backward TemplateParams
// entry: the chain starts with the dO.O row dot product, then the main pass
// and the dQ pass).
//
// Two kernels, in order on one stream, no atomics (bit-identical results
// run to run):
//   bwd_dq    one wave per 32 queries: its Q and dO rows stay in VGPRs, and
//             64-key tiles of K, V stream through LDS. Each lane first forms
//             its query's D = rowsum(dO * O) from its dO row and the O row,
//             and LSE in base 2 (LSE * log2 e; +inf for a row without
//             visible keys so that its P is 0), and writes both to the
//             workspace. Per tile: S^T = K Q^T and dP^T = V dO^T (the lane
//             owns one query), dS^T in VGPRs, then dQ^T += K^T dS^T;
//   bwd_dkdv  one wave per 32 keys of one K/V head: its K and V rows stay in
//             VGPRs as MFMA B operands, and 64-query tiles of Q, dO (with
//             their LSE and D) of every query head that reads this K/V head
//             stream through double-buffered LDS, so dK and dV sum over the
//             head group in registers. Per tile: S = Q K^T and dP = dO V^T
//             (the lane owns one key column), P and dS in VGPRs, then
//             dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read
//             through the transposing LDS read ds_read_b64_tr_b16.
// The contraction index of the second products is relabelled exactly as in
// the forward (P, dS go from the MFMA C layout to B operands in registers).
//
// Masking follows the forward's band (cudnn-frontend PR #554's sdpa API:
// is_causal, causal_bottom_right, window_left): query i of a sequence with
// s_q queries and s_kv keys sits on diagonal key p = i (+ s_kv - s_q when
// aligned bottom-right) and sees keys p - W .. p (no upper bound without
// causal, no lower one without a window). Each workgroup visits only the
// tiles that intersect the band, each wave skips the tiles its rows or keys
// do not reach, and element masks run only on tiles the band cuts. Query
// head i reads K/V head i / (h / h_kv). The packed (THD) variant takes each
// sequence's lengths from cu_seqlens; its statistic and workspace rows are
// token-major (token * h + head).

#include <mutex>

#include "kernel_common.h"
#include "sdpa_internal.h"

namespace sdpa07 {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBwdThreads = 256;
constexpr int kDkdvThreads = 512;  // four wave pairs
constexpr int kDkdvKeys = 128;  // keys per dK/dV workgroup (32 per wave pair)
constexpr int kDkdvQ = 64;      // queries per streamed tile
constexpr int kDqRows = 128;    // queries per dQ workgroup (32 per wave)
constexpr int kDqK = 64;        // keys per streamed tile
constexpr int kNoWindow = 1 << 29;  // window_left = -1: a left bound no key reaches

template <typename T>
__device__ __forceinline__ float to_f(T x) {
  return (float)x;
}

// Rows of one batch entry (dense) or one packed sequence (THD): lengths and
// the element offsets of its row 0 for a given head. Packed bounds are
// clamped to [0, total) so rows past the packed totals are never touched.
template <bool VARLEN>
struct Seq {
  int bi, q0, k0, q_len, kv_len;
  __device__ Seq(const BwdParams& p, int b) : bi(b) {
    if constexpr (VARLEN) {
      q0 = min(max(p.cu_q[b], 0), p.total_q);
      const int q1 = min(max(p.cu_q[b + 1], 0), p.total_q);
      k0 = min(max(p.cu_kv[b], 0), p.total_kv);
      const int k1 = min(max(p.cu_kv[b + 1], 0), p.total_kv);
      q_len = max(q1 - q0, 0);
      kv_len = max(k1 - k0, 0);
    } else {
      q0 = k0 = 0;
      q_len = p.s_q;
      kv_len = p.s_kv;
    }
  }
  __device__ int64_t qoff(int64_t sb, int64_t sh, int64_t ss, int hd) const {
    return (VARLEN ? (int64_t)q0 * ss : (int64_t)bi * sb) + (int64_t)hd * sh;
  }
  __device__ int64_t koff(int64_t sb, int64_t sh, int64_t ss, int hd) const {
    return (VARLEN ? (int64_t)k0 * ss : (int64_t)bi * sb) + (int64_t)hd * sh;
  }
  // index of query row 0 of head hd in the statistic / workspace rows, and
  // the step between consecutive query rows
  __device__ int64_t st0(const BwdParams& p, int hd) const {
    return VARLEN ? (int64_t)q0 * p.h + hd : ((int64_t)bi * p.h + hd) * p.s_q;
  }
  static __device__ int st_step(const BwdParams& p) { return VARLEN ? p.h : 1; }
};

// ---------------------------------------------------------------------------
// The dK/dV pass's Q and dO tiles in LDS: rows of D elements, unpadded,
// whose 16-byte chunks are permuted by an XOR of the row index (only r mod
// 16 matters), so that both ways a tile is read hit distinct banks: the MFMA
// row-operand reads (ds_read_b128, 16 rows per phase) and the transposing
// reads (ds_read_b64_tr_b16, 4 rows x 64 B per 32 lanes). No row padding
// serves both: the first needs a row stride of an odd number of 16-byte
// groups modulo 256 B, the second one of 64 B. Logical chunk c of row r
// sits at chunk c ^ tile_swz<D>(r).
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  return D <= 64 ? (((r >> 1) ^ (((r >> 1) & 1) << 2)) & 7) : ((r ^ ((r & 3) << 2)) & 15);
}

// Row-operand read: row r, logical chunk ch (8 elements), with s = tile_swz(r).
template <typename T, int D>
__device__ __forceinline__ typename Mfma16<T>::v8 read_row(const T* base, int r, int ch, int s) {
  return *(const typename Mfma16<T>::v8*)&base[r * D + ((ch ^ s) << 3)];
}

// Transposing LDS read of an A operand: lane (16-group g, index i) receives
// rows rbase + 4hf + 0..3 and + 8 .. 11 of column cbase + 16(g%2) + i
// (row = rbase + 4hf + (i / 4); s0, s1: tile_swz of row and of row + 8).
template <typename T, int D>
__device__ __forceinline__ typename Mfma16<T>::v8 read_tr(const T* base, int row, int colv, int s0,
                                                          int s1) {
  const T* a0 = base + row * D + (((colv >> 3) ^ s0) << 3) + (colv & 7);
  const T* a1 = base + (row + 8) * D + (((colv >> 3) ^ s1) << 3) + (colv & 7);
  const i16x4 lo =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(a0));
  const i16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(a1));
  return __builtin_bit_cast(typename Mfma16<T>::v8,
                            __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Packs 32 fp32 values held in a [2] x 16 MFMA C layout into 4 B operands
// for a 64-deep contraction (element e of MFMA t: register 8(t%2)+e of block t/2).
template <typename T>
__device__ __forceinline__ void pack_b(const f32x16 (&x)[2], typename Mfma16<T>::v8 (&out)[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    i32x4 pk;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const f32x2 v = {x[t / 2][8 * (t % 2) + 2 * e2], x[t / 2][8 * (t % 2) + 2 * e2 + 1]};
      pk[e2] = __builtin_bit_cast(int, __builtin_convertvector(v, typename Pack2<T>::type));
    }
    out[t] = __builtin_bit_cast(typename Mfma16<T>::v8, pk);
  }
}

// The same for one 32-key block: 16 values into the 2 B operands of a
// 32-deep contraction (element e of MFMA t: register 8t + e).
template <typename T>
__device__ __forceinline__ void pack_b1(const f32x16& x, typename Mfma16<T>::v8 (&out)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    i32x4 pk;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const f32x2 v = {x[8 * t + 2 * e2], x[8 * t + 2 * e2 + 1]};
      pk[e2] = __builtin_bit_cast(int, __builtin_convertvector(v, typename Pack2<T>::type));
    }
    out[t] = __builtin_bit_cast(typename Mfma16<T>::v8, pk);
  }
}

// ---------------------------------------------------------------------------
// dK/dV: a pair of waves owns 32 keys of one K/V head, and the workgroup's
// four pairs own 128 consecutive keys. The first wave of a pair (K side)
// keeps the K rows of its keys as MFMA B operands; per query tile it computes
// S = Q K^T and P, accumulates dV^T += dO^T P and leaves P in LDS (fp32, in
// the C layout both waves share). Its partner (V side) keeps the V rows and
// runs one tile behind: it finishes the previous tile's dS = P (dP - D) with
// the P its partner left there and accumulates dK^T += Q^T dS, then computes
// this tile's dP = dO V^T. Each wave thus needs half the registers of one
// that does both sides, so two waves share a SIMD and hide each other's LDS
// and MFMA latencies; both do 32 MFMAs per tile, and one barrier per tile
// orders them. 64-query tiles of Q (three buffers, as the V side reads the
// previous one), dO (two) and their LSE and D of every query head that reads
// this K/V head stream through LDS, so dK and dV sum over the head group in
// registers.
template <typename T, int D, bool CAUSAL, bool VARLEN>
__global__ void __launch_bounds__(kDkdvThreads) __attribute__((amdgpu_waves_per_eu(2)))
bwd_dkdv_kernel(BwdParams p, const float* lse2) {
  constexpr int BQ = kDkdvQ;
  using M = Mfma16<T>;
  using v8 = typename M::v8;
  __shared__ __attribute__((aligned(16))) T ql[3][BQ * D];
  __shared__ __attribute__((aligned(16))) T gl[2][BQ * D];
  __shared__ __attribute__((aligned(16))) float l2l[2][BQ];
  __shared__ __attribute__((aligned(16))) float dll[2][BQ];
  // P of each pair and tile parity: [query block][register quad][lane][4]
  __shared__ __attribute__((aligned(16))) float pl[2][4][2 * 4 * 64 * 4];

  // Dense: blockIdx -> (key tile, b*h_kv), the first key tiles (which a
  // causal band shows to the most queries) first. Packed: blockIdx -> (live
  // key tile of a sequence, K/V head), heads innermost, the tiles of all
  // sequences in decreasing order of work (causal without a left bound: key
  // tile t of a sequence costs n - t; other masks: the query count).
  int kt, bi, hk;
  if constexpr (VARLEN) {
    hk = blockIdx.x % p.h_kv;
    const bool taper = CAUSAL && p.window_left < 0;
    const PackedUnit pu = packed_unit(blockIdx.x / p.h_kv, p.b, taper, [&](int s) -> int2 {
      const int nk = (packed_len(p.cu_kv, s, p.total_kv) + kDkdvKeys - 1) / kDkdvKeys;
      if (taper) return int2{nk, nk};
      return int2{nk, max((packed_len(p.cu_q, s, p.total_q) + kDkdvQ - 1) / kDkdvQ, 1)};
    });
    if (pu.seq < 0) return;  // past the last key tile (uniform over the workgroup)
    bi = pu.seq;
    kt = pu.j;
  } else {
    const int nbh = p.b * p.h_kv;
    kt = blockIdx.x / nbh;
    const int bh = blockIdx.x % nbh;
    bi = bh / p.h_kv;
    hk = bh % p.h_kv;
  }
  const int group = p.h / p.h_kv;  // query heads hk * group .. + group - 1 read this K/V head
  const Seq<VARLEN> sq(p, bi);
  if (kt * kDkdvKeys >= sq.kv_len) return;
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int pair = wave % 4;
  const bool kside = wave < 4;
  const int hf = lane / 32, col = lane % 32;
  const int key0 = kt * kDkdvKeys + pair * 32;  // first key of this pair
  const int kj = key0 + col;                     // this lane's key
  const int shift = p.bottom_right ? sq.kv_len - sq.q_len : 0;
  const int window = p.window_left < 0 ? kNoWindow : p.window_left;
  const float c = p.scale_log2;
  const int st_step = Seq<VARLEN>::st_step(p);

  // this lane's K (or V) row as B operands (B[k = d][n = key])
  const T* R = kside ? (const T*)p.k + sq.koff(p.k_sb, p.k_sh, p.k_ss, hk)
                     : (const T*)p.v + sq.koff(p.v_sb, p.v_sh, p.v_ss, hk);
  const int64_t r_ss = kside ? p.k_ss : p.v_ss;
  v8 bf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    i16x8 a = {};
    if (kj < sq.kv_len) a = *(const i16x8*)(R + (int64_t)kj * r_ss + 16 * ks + 8 * hf);
    bf[ks] = __builtin_bit_cast(v8, a);
  }
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

  // Query rows that see a key of this workgroup: i + shift >= first key
  // (causal) and i + shift - window <= last key.
  const int key_hi = min(sq.kv_len, kt * kDkdvKeys + kDkdvKeys) - 1;
  const int i_lo = CAUSAL ? max(kt * kDkdvKeys - shift, 0) : 0;
  const int i_hi = min(sq.q_len - 1, key_hi - shift + window);
  const int t_lo = i_lo / BQ;
  const int nt = i_hi >= i_lo ? i_hi / BQ + 1 - t_lo : 0;  // query tiles per head
  // the tiles this pair's keys reach (inclusive bounds)
  const int wt_lo = CAUSAL ? max(key0 - shift, 0) / BQ : 0;
  const int wi_hi = min(key0 + 31, sq.kv_len - 1) - shift + window;
  const int wt_hi = key0 < sq.kv_len && wi_hi >= 0 ? wi_hi / BQ : -1;

  // iteration it covers query head hk * group + it / nt, tile t_lo + it % nt
  const int n_it = group * nt;
  // Q and dO tiles go from memory straight into LDS (buffer loads with the
  // LDS flag) in unpadded rows with the chunk swizzle: load instruction x of
  // wave w fills rows RIT(x) .. RIT(x) + RPI - 1 (1 KB), lane l row
  // RIT(x) + l / CH, slot l % CH, with the global chunk that the slot holds.
  // Rows past the sequence read as zeros (the descriptor's byte bound).
  constexpr int CH = D / 8;               // 16-byte chunks per row
  constexpr int RPI = 64 / CH;            // rows per load instruction
  constexpr int NW = kDkdvThreads / 64;   // waves
  constexpr int CPT = BQ / (RPI * NW);    // load instructions per wave per tensor
  static_assert(CPT >= 1 && BQ % (RPI * NW) == 0, "tile/workgroup mismatch");
  static_assert((NW * RPI) % 16 == 0, "load rows change the swizzle phase");
  auto RIT = [&](int x) { return (NW * x + wave) * RPI; };
  const int drow = lane / CH;
  const int dch = (lane % CH) ^ tile_swz<D>((RIT(0) + drow) % 16);  // RIT(x) mod 16: same for all x
  const int qvoff = drow * (int)p.q_ss * (int)sizeof(T) + dch * 16;
  const int gvoff = drow * (int)p.do_ss * (int)sizeof(T) + dch * 16;
  auto tile_rsrc = [&](const T* tile, int64_t stride, int rows) -> i32x4 {
    const int bytes = rows <= 0 ? 0 : ((min(rows, BQ) - 1) * (int)stride + D) * (int)sizeof(T);
    const unsigned long long a = (unsigned long long)tile;
    return i32x4{(int)(unsigned)a, (int)((unsigned)(a >> 32) & 0xffffu), bytes, kBufferFlags};
  };
  auto lds_addr = [](const T* x) {
    return (unsigned)(size_t)(__attribute__((address_space(3))) const T*)x;
  };
  float l2r = 0.f, dlr = 0.f;
  // tile t of query head hq into Q buffer qslot and dO buffer gslot (the
  // iterations step through the tiles of each head in turn; the loops keep
  // (head, tile) counters, no divisions)
  auto gload = [&](int hq, int t, int qslot, int gslot) {
    const int rows = sq.q_len - t * BQ;
    const i32x4 rq =
        tile_rsrc((const T*)p.q + sq.qoff(p.q_sb, p.q_sh, p.q_ss, hq) + (int64_t)t * BQ * p.q_ss,
                  p.q_ss, rows);
    const i32x4 rg = tile_rsrc(
        (const T*)p.dout + sq.qoff(p.do_sb, p.do_sh, p.do_ss, hq) + (int64_t)t * BQ * p.do_ss,
        p.do_ss, rows);
#pragma unroll
    for (int x = 0; x < CPT; ++x)
      lds_dma16(rq, qvoff, RIT(x) * (int)p.q_ss * (int)sizeof(T),
                lds_addr(ql[qslot] + RIT(x) * D));
#pragma unroll
    for (int x = 0; x < CPT; ++x)
      lds_dma16(rg, gvoff, RIT(x) * (int)p.do_ss * (int)sizeof(T),
                lds_addr(gl[gslot] + RIT(x) * D));
    if (tid < BQ) {
      const int qrow = t * BQ + tid;
      const int64_t si = sq.st0(p, hq) + (int64_t)qrow * st_step;
      l2r = qrow < sq.q_len ? lse2[si] : INFINITY;
      dlr = qrow < sq.q_len ? p.delta[si] : 0.f;
    }
  };
  auto lstore = [&](int it) {  // the tile's statistic and D
    if (tid < BQ) {
      l2l[it & 1][tid] = l2r;
      dll[it & 1][tid] = dlr;
    }
  };
  auto active = [&](int t) {  // the pair's keys see query tile t (the same for both waves)
    return t >= wt_lo && t <= wt_hi;
  };
  // (head, tile) of the next iteration, from the current one
  auto next = [&](int& h, int& t) {
    if (++t == t_lo + nt) {
      t = t_lo;
      ++h;
    }
  };
  const int vrow = 4 * hf + (lane % 16) / 4;
  const int vcol = 16 * ((lane / 16) % 2) + 4 * (lane % 4);
  // chunk permutations of the rows this lane reads (rows 32qb + col and
  // 16t + vrow (+ 8) share those of col and vrow)
  const int sr = tile_swz<D>(col % 16), st0 = tile_swz<D>(vrow), st1 = tile_swz<D>(vrow + 8);
  // acc += A2^T X over the 64 queries of a tile, A2^T read through the
  // transposing LDS read (dO^T for dV, Q^T for dK)
  auto accumulate = [&](const T* a2, const f32x16 (&x)[2]) {
    v8 xb[4];
    pack_b<T>(x, xb);
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const v8 a = read_tr<T, D>(a2, 16 * t4 + vrow, 32 * db + vcol, st0, st1);
        acc[db] = M::mma(a, xb[t4], acc[db]);
      }
  };
  // x = A1 B over the d columns, A1 rows read from LDS (Q for S, dO for dP);
  // C layout: lane = key kj, register r of block qb = query
  // t*BQ + 32qb + 8(r/4) + 4hf + r%4
  auto product = [&](const T* a1, f32x16 (&x)[2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      x[qb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const v8 a = read_row<T, D>(a1, 32 * qb + col, 2 * ks + hf, sr);
        x[qb] = M::mma(a, bf[ks], x[qb]);
      }
    }
  };

  if (n_it > 0) {
    gload(hk * group, t_lo, 0, 0);
    lstore(0);
  }
  // Every load issued so far (the B-operand rows above all) has landed on
  // every path into the loop; without this the compiler cannot tell, and
  // waits for all outstanding loads, the next tile's included, at their
  // first use in each iteration.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // Both loops run n_it + 1 steps with one barrier each; tile it sits in Q
  // buffer it % 3 (kept as qs) and in the other buffers at parity it & 1.
  if (kside) {
    f32x16 x[2];
    int tc = t_lo, hn = hk * group, tn = t_lo;  // tile of iteration it; head, tile of it + 1
    next(hn, tn);
    for (int it = 0, qs = 0; it <= n_it; ++it) {
      const int qn = qs == 2 ? 0 : qs + 1;
      if (it + 1 < n_it) gload(hn, tn, qn, (it + 1) & 1);  // buffers free since the last barrier
      if (it < n_it && active(tc)) {
        product(ql[qs], x);  // S = Q K^T
        const int q_first = tc * BQ;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const float4 l4 = *(const float4*)&l2l[it & 1][32 * qb + 8 * rq + 4 * hf];
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              x[qb][4 * rq + e] = fast_exp2(fmaf(x[qb][4 * rq + e], c, -lv[e]));
          }
        // The band cuts the tile at the causal edge if its first query hides
        // the pair's last key, at the window's edge if its last query hides
        // the pair's first key. Query 32qb + 8rq + e (+ q_first + 4hf) hides
        // key kj when causal and kj > query + shift, or kj < query + shift - W.
        if (CAUSAL && key0 + 31 > q_first + shift) {
          const int lim = kj - shift - q_first - 4 * hf;
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              x[qb][r] = 32 * qb + 8 * (r / 4) + r % 4 < lim ? 0.f : x[qb][r];
        }
        if (key0 < q_first + BQ - 1 + shift - window) {
          const int lim = kj - shift + window - q_first - 4 * hf;
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              x[qb][r] = 32 * qb + 8 * (r / 4) + r % 4 > lim ? 0.f : x[qb][r];
        }
        float* pp = pl[it & 1][pair];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq)
            *(float4*)&pp[((qb * 4 + rq) * 64 + lane) * 4] =
                float4{x[qb][4 * rq], x[qb][4 * rq + 1], x[qb][4 * rq + 2], x[qb][4 * rq + 3]};
        accumulate(gl[it & 1], x);  // dV^T += dO^T P
      }
      if (it + 1 < n_it) lstore(it + 1);
      // this wave's tile loads have landed; after the barrier every wave's
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      qs = qn;
      tc = tn;
      next(hn, tn);
    }
  } else {
    f32x16 x[2];  // dP - D of the previous tile
    // tiles of iterations it - 1 and it; head, tile of it + 1
    int tp = -1, tc = t_lo, hn = hk * group, tn = t_lo;
    next(hn, tn);
    for (int it = 0, qs = 0, qp = 2; it <= n_it; ++it) {
      const int qn = qs == 2 ? 0 : qs + 1;
      if (it + 1 < n_it) gload(hn, tn, qn, (it + 1) & 1);  // buffers free since the last barrier
      if (it > 0 && active(tp)) {
        // dS = P (dP - D) of the previous tile, then dK^T += Q^T dS
        const float* pp = pl[(it - 1) & 1][pair];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const float4 p4 = *(const float4*)&pp[((qb * 4 + rq) * 64 + lane) * 4];
            x[qb][4 * rq] = p4.x * x[qb][4 * rq];
            x[qb][4 * rq + 1] = p4.y * x[qb][4 * rq + 1];
            x[qb][4 * rq + 2] = p4.z * x[qb][4 * rq + 2];
            x[qb][4 * rq + 3] = p4.w * x[qb][4 * rq + 3];
          }
        accumulate(ql[qp], x);
      }
      if (it < n_it && active(tc)) {
        product(gl[it & 1], x);  // dP = dO V^T
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const float4 d4 = *(const float4*)&dll[it & 1][32 * qb + 8 * rq + 4 * hf];
            const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) x[qb][4 * rq + e] -= dd[e];
          }
      }
      if (it + 1 < n_it) lstore(it + 1);
      // this wave's tile loads have landed; after the barrier every wave's
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      qp = qs;
      qs = qn;
      tp = tc;
      tc = tn;
      next(hn, tn);
    }
  }

  // store: lane owns key kj, d rows 32db + 8rq + 4hf + 0..3; the rows go
  // whole through the wave's part of the P exchange (every wave is past the
  // loops' last barrier)
  const int64_t out_ss = kside ? p.dv_ss : p.dk_ss;
  if (out_ss < (1 << 24)) {
    static_assert(kDkdvThreads / 64 * 32 * D * (int)sizeof(T) <= (int)sizeof(pl),
                  "staging rows exceed the P exchange");
    T* dst0 = kside ? (T*)p.dv + sq.koff(p.dv_sb, p.dv_sh, p.dv_ss, hk) + (int64_t)key0 * p.dv_ss
                    : (T*)p.dk + sq.koff(p.dk_sb, p.dk_sh, p.dk_ss, hk) + (int64_t)key0 * p.dk_ss;
    store_rows_via_lds<T, D>((T*)&pl[0][0][0] + wave * 32 * D, acc, kside ? 1.f : p.scale, dst0,
                             out_ss, sq.kv_len - key0, lane);
  } else if (kj < sq.kv_len) {
    T* dst = kside ? (T*)p.dv + sq.koff(p.dv_sb, p.dv_sh, p.dv_ss, hk) + (int64_t)kj * p.dv_ss
                   : (T*)p.dk + sq.koff(p.dk_sb, p.dk_sh, p.dk_ss, hk) + (int64_t)kj * p.dk_ss;
    const float f = kside ? 1.f : p.scale;
    typedef T t4v __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        t4v a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = (T)(acc[db][4 * rq + e] * f);
        *(t4v*)(dst + 32 * db + 8 * rq + 4 * hf) = a;
      }
  }
}

// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL, bool VARLEN>
__global__ void __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2)))
bwd_dq_kernel(BwdParams p, float* lse2) {
  // K and V tiles go from memory straight into double-buffered LDS (buffer
  // loads with the LDS flag, no staging registers), in unpadded rows whose
  // 16-byte chunks carry the chunk swizzle: the row reads (S^T, dP^T) and
  // the transposing reads (K^T) are both free of bank conflicts.
  constexpr int BK = kDqK;
  using M = Mfma16<T>;
  using v8 = typename M::v8;
  __shared__ __attribute__((aligned(16))) T kl[2][BK * D];
  __shared__ __attribute__((aligned(16))) T vl[2][BK * D];

  // Dense: blockIdx -> (query tile, b*h), the heaviest causal tiles first.
  // Packed: blockIdx -> (live query tile of a sequence, head), heads
  // innermost, the tiles of all sequences in decreasing order of work
  // (causal without a left bound: tile t costs t + 1; other masks: the keys).
  int qt, bi, hi;
  if constexpr (VARLEN) {
    hi = blockIdx.x % p.h;
    const bool taper = CAUSAL && p.window_left < 0;
    const PackedUnit pu = packed_unit(blockIdx.x / p.h, p.b, taper, [&](int s) -> int2 {
      const int nq = (packed_len(p.cu_q, s, p.total_q) + kDqRows - 1) / kDqRows;
      if (taper) return int2{nq, nq};
      return int2{nq, max((packed_len(p.cu_kv, s, p.total_kv) + kDqK - 1) / kDqK, 1)};
    });
    if (pu.seq < 0) return;  // past the last query tile (uniform over the workgroup)
    bi = pu.seq;
    const int nq = (packed_len(p.cu_q, bi, p.total_q) + kDqRows - 1) / kDqRows;
    qt = taper ? nq - 1 - pu.j : pu.j;
  } else {
    const int nbh = p.b * p.h;
    const int n_qtiles = (p.s_q + kDqRows - 1) / kDqRows;
    qt = n_qtiles - 1 - (int)(blockIdx.x / nbh);  // heaviest causal tiles first
    const int bh = blockIdx.x % nbh;
    bi = bh / p.h;
    hi = bh % p.h;
  }
  const int hk = hi / (p.h / p.h_kv);  // K/V head of this query head
  const Seq<VARLEN> sq(p, bi);
  if (qt * kDqRows >= sq.q_len) return;
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int hf = lane / 32, col = lane % 32;
  const int row0 = qt * kDqRows + wave * 32;
  const int qi = row0 + col;
  const bool q_valid = qi < sq.q_len;
  const int shift = p.bottom_right ? sq.kv_len - sq.q_len : 0;
  const int window = p.window_left < 0 ? kNoWindow : p.window_left;

  const T* Q = (const T*)p.q + sq.qoff(p.q_sb, p.q_sh, p.q_ss, hi);
  const T* G = (const T*)p.dout + sq.qoff(p.do_sb, p.do_sh, p.do_ss, hi);
  const T* K = (const T*)p.k + sq.koff(p.k_sb, p.k_sh, p.k_ss, hk);
  const T* V = (const T*)p.v + sq.koff(p.v_sb, p.v_sh, p.v_ss, hk);
  const float c = p.scale_log2;
  const int64_t si = sq.st0(p, hi) + (int64_t)qi * Seq<VARLEN>::st_step(p);

  v8 qf[D / 16], gf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    i16x8 a = {}, b = {};
    if (q_valid) {
      a = *(const i16x8*)(Q + (int64_t)qi * p.q_ss + 16 * ks + 8 * hf);
      b = *(const i16x8*)(G + (int64_t)qi * p.do_ss + 16 * ks + 8 * hf);
    }
    qf[ks] = __builtin_bit_cast(v8, a);
    gf[ks] = __builtin_bit_cast(v8, b);
  }
  // this lane's query: D = rowsum(dO * O) (the two lane halves hold
  // alternate 8-column chunks of the row) and the statistic in base 2 (+inf
  // for a row that sees no key, so that its P is 0); both also go to the
  // workspace for the dK/dV pass, which runs after this one
  float dpart = 0.f;
  if (q_valid) {
    const T* Orow = (const T*)p.o + sq.qoff(p.o_sb, p.o_sh, p.o_ss, hi) + (int64_t)qi * p.o_ss;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const v8 o8 = __builtin_bit_cast(v8, *(const i16x8*)(Orow + 16 * ks + 8 * hf));
#pragma unroll
      for (int e = 0; e < 8; ++e) dpart = fmaf(to_f(o8[e]), to_f(gf[ks][e]), dpart);
    }
  }
  const float dl = dpart + other_half(dpart);
  const float lraw = q_valid ? p.lse[si] : -INFINITY;
  const float l2 = lraw == -INFINITY ? INFINITY : lraw * kLog2e;
  if (q_valid && hf == 0) {
    p.delta[si] = dl;
    lse2[si] = l2;
  }
  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = f32x16{};

  // keys of the workgroup's band: [kv_begin, kv_end)
  const int last_q = min(sq.q_len, (qt + 1) * kDqRows) - 1;
  const int kv_end = CAUSAL ? min(sq.kv_len, max(last_q + shift + 1, 0)) : sq.kv_len;
  const int kv_begin = min(kv_end, max(qt * kDqRows + shift - window, 0));
  const int j0 = kv_begin / BK;
  const int j1 = kv_end > kv_begin ? (kv_end + BK - 1) / BK : j0;
  // the wave's band: keys [wave_kv_begin, wave_kv_end)
  const int w_last = min(sq.q_len, row0 + 32) - 1;
  const int wave_kv_end =
      row0 >= sq.q_len ? 0 : (CAUSAL ? min(sq.kv_len, w_last + shift + 1) : sq.kv_len);
  const int wave_kv_begin = row0 + shift - window;
  // Load instruction x of wave w fills rows RIT(x) .. RIT(x) + RPI - 1 of a
  // tile (1 KB of LDS); lane l fills row RIT(x) + l / CH, slot l % CH, with
  // the global chunk that the slot holds under the row's swizzle. Rows past
  // the keys read as zeros (the descriptor's byte bound ends with the last
  // key row).
  constexpr int CH = D / 8;             // 16-byte chunks per row
  constexpr int RPI = 64 / CH;          // rows per load instruction
  constexpr int NW = kBwdThreads / 64;  // waves
  constexpr int CPT = BK / (RPI * NW);  // load instructions per wave per tensor
  static_assert(CPT >= 1 && BK % (RPI * NW) == 0, "tile/workgroup mismatch");
  static_assert((NW * RPI) % 16 == 0, "load rows change the swizzle phase");
  auto RIT = [&](int x) { return (NW * x + wave) * RPI; };
  const int drow = lane / CH;
  const int dch = (lane % CH) ^ tile_swz<D>((RIT(0) + drow) % 16);  // RIT(x) mod 16: same for all x
  const int kvoff = drow * (int)p.k_ss * (int)sizeof(T) + dch * 16;
  const int vvoff = drow * (int)p.v_ss * (int)sizeof(T) + dch * 16;
  auto tile_rsrc = [&](const T* base, int64_t stride, int j) -> i32x4 {
    const int rows = min(sq.kv_len - j * BK, BK);
    const int bytes = rows <= 0 ? 0 : ((rows - 1) * (int)stride + D) * (int)sizeof(T);
    const unsigned long long a = (unsigned long long)(base + (int64_t)j * BK * stride);
    return i32x4{(int)(unsigned)a, (int)((unsigned)(a >> 32) & 0xffffu), bytes, kBufferFlags};
  };
  auto lds_addr = [](const T* x) {
    return (unsigned)(size_t)(__attribute__((address_space(3))) const T*)x;
  };
  auto gload = [&](int j, int buf) {
    const i32x4 rk = tile_rsrc(K, p.k_ss, j), rv = tile_rsrc(V, p.v_ss, j);
#pragma unroll
    for (int x = 0; x < CPT; ++x)
      lds_dma16(rk, kvoff, RIT(x) * (int)p.k_ss * (int)sizeof(T), lds_addr(kl[buf] + RIT(x) * D));
#pragma unroll
    for (int x = 0; x < CPT; ++x)
      lds_dma16(rv, vvoff, RIT(x) * (int)p.v_ss * (int)sizeof(T), lds_addr(vl[buf] + RIT(x) * D));
  };
  const int vrow = 4 * hf + (lane % 16) / 4;
  const int vcol = 16 * ((lane / 16) % 2) + 4 * (lane % 4);
  // chunk permutations of the rows this lane reads: rows 32kb + col for
  // S^T and dP^T, rows 16t + vrow (+ 8) for the transposing K^T reads
  const int sk = tile_swz<D>(col % 16), sk0 = tile_swz<D>(vrow), sk1 = tile_swz<D>(vrow + 8);

  if (j1 > j0) gload(j0, 0);
  // The Q, dO rows above and the first tile have landed in every wave
  // before the loop (the compiler cannot see the tile loads' completion).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int j = j0; j < j1; ++j) {
    const int buf = (j - j0) & 1;
    if (j + 1 < j1) gload(j + 1, buf ^ 1);  // every wave is done with buf ^ 1
    const int kbase = j * BK;
    if (kbase < wave_kv_end && kbase + BK > wave_kv_begin) {
      const T* kb_ = kl[buf];
      const T* vb_ = vl[buf];
      // The band cuts the tile at the causal edge if the wave's first query
      // hides the tile's last key, at the window's edge if its last query
      // hides the tile's first key, and at the end of the keys.
      const bool cut_causal = CAUSAL && kbase + BK - 1 > row0 + shift;
      const bool cut_left = kbase < w_last + shift - window;
      const bool cut_end = kbase + BK > sq.kv_len;
      // The tile's two 32-key blocks one after the other (fewer live
      // registers): S^T = K Q^T and dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
      // Lane = query qi; register r of block kb = key
      // kbase + 32kb + 8(r/4) + 4hf + r%4.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 sv = {}, dp = {};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const v8 ak = read_row<T, D>(kb_, 32 * kb + col, 2 * ks + hf, sk);
          const v8 av = read_row<T, D>(vb_, 32 * kb + col, 2 * ks + hf, sk);
          sv = M::mma(ak, qf[ks], sv);
          dp = M::mma(av, gf[ks], dp);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[r] = fast_exp2(fmaf(sv[r], c, -l2));
        // key offset 32kb + 8(r/4) + r%4 (+ kbase + 4hf) against each bound
        const int base = kbase + 32 * kb + 4 * hf;
        if (CAUSAL && cut_causal) {
          const int lim = qi + shift - base;
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[r] = 8 * (r / 4) + r % 4 > lim ? 0.f : sv[r];
        }
        if (cut_left) {
          const int lim = qi + shift - window - base;
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[r] = 8 * (r / 4) + r % 4 < lim ? 0.f : sv[r];
        }
        if (cut_end) {
          const int lim = sq.kv_len - base;
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[r] = 8 * (r / 4) + r % 4 >= lim ? 0.f : sv[r];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = sv[r] * (dp[r] - dl);
        v8 sb[2];
        pack_b1<T>(dp, sb);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const v8 ak = read_tr<T, D>(kb_, 16 * (2 * kb + t) + vrow, 32 * db + vcol, sk0, sk1);
            dq[db] = M::mma(ak, sb[t], dq[db]);
          }
      }
    }
    // this wave's loads of tile j + 1 have landed; after the barrier every
    // wave's have, and every wave is done with buffer buf
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // dQ rows whole through the wave's part of the K buffers (every wave is
  // past the loop's last barrier)
  if (p.dq_ss < (1 << 24)) {
    static_assert(kBwdThreads / 64 * 32 * D * (int)sizeof(T) <= (int)sizeof(kl),
                  "staging rows exceed the K buffers");
    T* dq0 = (T*)p.dq + sq.qoff(p.dq_sb, p.dq_sh, p.dq_ss, hi) + (int64_t)max(row0, 0) * p.dq_ss;
    store_rows_via_lds<T, D>((T*)&kl[0][0] + wave * 32 * D, dq, p.scale, dq0, p.dq_ss,
                             sq.q_len - row0, lane);
  } else if (q_valid) {
    T* dqp = (T*)p.dq + sq.qoff(p.dq_sb, p.dq_sh, p.dq_ss, hi) + (int64_t)qi * p.dq_ss;
    typedef T t4v __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        t4v a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = (T)(dq[db][4 * rq + e] * p.scale);
        *(t4v*)(dqp + 32 * db + 8 * rq + 4 * hf) = a;
      }
  }
}

// Fills a dense (b, h, s, d) tensor with zeros (dK, dV when there are no
// queries, dQ when there are no keys).
template <typename T, int D>
__global__ void __launch_bounds__(256) zero_rows_kernel(void* x, int64_t sb, int64_t sh,
                                                        int64_t ss, int b, int h, int s) {
  const long long r = (long long)blockIdx.x * (256 / (D / 8)) + threadIdx.x / (D / 8);
  const int sub = threadIdx.x % (D / 8);
  if (r >= (long long)b * h * s) return;
  const int si = (int)(r % s);
  const long long bh = r / s;
  T* ptr = (T*)x + (bh / h) * sb + (bh % h) * sh + (int64_t)si * ss + sub * 8;
  *(i16x8*)ptr = i16x8{};
}

template <typename T, int D>
hipError_t zero_rows(void*& x, int64_t& sb, int64_t& sh, int64_t& ss, int& b, int& h, int& s,
                     hipStream_t stream) {
  const long long rows = (long long)b * h * s;
  const int per = 256 / (D / 8);
  const dim3 g((unsigned)((rows + per - 1) / per));
  void* a[] = {&x, &sb, &sh, &ss, &b, &h, &s};
  return hipLaunchKernel((const void*)&zero_rows_kernel<T, D>, g, dim3(256), a, 0, stream);
}

template <typename T, int D, bool CAUSAL, bool VARLEN>
hipError_t launch_typed(const BwdParams& p, hipStream_t stream) {
  BwdParams arg = p;
  const long long n = VARLEN ? (long long)p.total_q * p.h : (long long)p.b * p.h * p.s_q;
  hipError_t e;
  if (!VARLEN && (p.s_q == 0 || p.s_kv == 0)) {
    // nothing to recompute: every gradient is zero
    if (p.s_kv > 0) {
      e = zero_rows<T, D>(arg.dk, arg.dk_sb, arg.dk_sh, arg.dk_ss, arg.b, arg.h_kv, arg.s_kv,
                          stream);
      if (e != hipSuccess) return e;
      return zero_rows<T, D>(arg.dv, arg.dv_sb, arg.dv_sh, arg.dv_ss, arg.b, arg.h_kv, arg.s_kv,
                             stream);
    }
    if (p.s_q > 0)
      return zero_rows<T, D>(arg.dq, arg.dq_sb, arg.dq_sh, arg.dq_ss, arg.b, arg.h, arg.s_q,
                             stream);
    return hipSuccess;
  }
  if (VARLEN && (p.total_q == 0 || p.total_kv == 0)) {
    // a packed batch with no keys (or no queries) anywhere: every gradient row
    // is zero, and O, dO, the statistic and the workspace are neither needed
    // nor read (the entry point does not require them in this case)
    int one = 1;
    int64_t no_sb = 0;
    if (p.total_kv > 0) {
      int rows = p.total_kv;
      e = zero_rows<T, D>(arg.dk, no_sb, arg.dk_sh, arg.dk_ss, one, arg.h_kv, rows, stream);
      if (e != hipSuccess) return e;
      return zero_rows<T, D>(arg.dv, no_sb, arg.dv_sh, arg.dv_ss, one, arg.h_kv, rows, stream);
    }
    if (p.total_q > 0) {
      int rows = p.total_q;
      return zero_rows<T, D>(arg.dq, no_sb, arg.dq_sh, arg.dq_ss, one, arg.h, rows, stream);
    }
    return hipSuccess;
  }
  // the workspace: D for every query row (padded to 64), then LSE in base 2,
  // both written by the dQ pass for every query row it covers (all of them)
  // and read by the dK/dV pass after it
  float* lse2 = p.delta + (n + 63) / 64 * 64;
  // packed sequences with no queries (or no keys) still get their dK, dV
  // (or dQ) rows written as zeros by these two kernels
  const long long gq = VARLEN ? packed_units_per_head(p.total_q, p.b, kDqRows) * p.h
                              : (long long)p.b * p.h * ((p.s_q + kDqRows - 1) / kDqRows);
  if (gq > 0) {
    void* args[] = {&arg, &lse2};
    e = hipLaunchKernel((const void*)&bwd_dq_kernel<T, D, CAUSAL, VARLEN>, dim3((unsigned)gq),
                        dim3(kBwdThreads), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  const long long gk =
      VARLEN ? packed_units_per_head(p.total_kv, p.b, kDkdvKeys) * p.h_kv
             : (long long)p.b * p.h_kv * ((p.s_kv + kDkdvKeys - 1) / kDkdvKeys);
  if (gk > 0) {
    void* args[] = {&arg, &lse2};
    e = hipLaunchKernel((const void*)&bwd_dkdv_kernel<T, D, CAUSAL, VARLEN>, dim3((unsigned)gk),
                        dim3(kDkdvThreads), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int D>
hipError_t launch_d(const BwdParams& p, bool causal, bool varlen, hipStream_t stream) {
  if (varlen)
    return causal ? launch_typed<T, D, true, true>(p, stream)
                  : launch_typed<T, D, false, true>(p, stream);
  return causal ? launch_typed<T, D, true, false>(p, stream)
                : launch_typed<T, D, false, false>(p, stream);
}

}  // namespace

size_t bwd_workspace_bytes(long long rows) {
  // D (rows floats, padded to 64) then LSE in base 2 (rows floats)
  const size_t n = (size_t)((rows + 63) / 64 * 64);
  return ((2 * n * sizeof(float)) + 255) / 256 * 256;
}

// The fixed workspace: a file-scope device array, so that the code object
// holds one copy per device from its load until the process ends. Host code
// never passes the array's name to a kernel (on the host that name is only a
// stand-in); it passes the device address looked up here.
static __device__ __align__(256) unsigned char scratch[kBwdFixedWorkspaceBytes];

hipError_t bwd_fixed_workspace(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_bwd(const BwdParams& p, Dt dt, int d, bool causal, bool varlen,
                      hipStream_t stream) {
  if (dt == Dt::BF16)
    return d == 64 ? launch_d<__bf16, 64>(p, causal, varlen, stream)
                   : launch_d<__bf16, 128>(p, causal, varlen, stream);
  if (dt == Dt::F16)
    return d == 64 ? launch_d<_Float16, 64>(p, causal, varlen, stream)
                   : launch_d<_Float16, 128>(p, causal, varlen, stream);
  return hipErrorInvalidValue;
}

}  // namespace sdpa07
