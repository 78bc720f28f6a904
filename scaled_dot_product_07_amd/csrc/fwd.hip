// Fused scaled-dot-product attention forward for gfx950 (MI355X).
//
// Computes O = softmax(scale * Q K^T + mask) V and the natural-log row
// statistic LSE for dense (b, h, s, d) batches and packed THD batches
// ("Inside NVIDIA's cuDNN Graph API ...", section 5: the operation, scale and
// top-left causal band; cudnn-frontend PR #554: statistic layouts and THD
// packing with cu_seqlens).
//
// fp16/bf16: query tiles of 128 rows go in pairs of one (b, h) or
// (sequence, h) (for a causal band without a left bound heavy with light,
// (n-1-i, i)), 32 rows per wave. At d = 64 and for causal bands each tile
// has a workgroup of its own (4 waves; 80 KB of LDS at d = 64, 64 KB at
// d = 128 where Q goes straight to registers; two per CU), and the grid puts
// the two tiles of a pair where the dispatcher places two workgroups on one
// CU, so that they share its SIMDs but not a barrier. Without a causal band
// at d = 128 one workgroup of 8 waves runs both tiles of a pair over one key
// stream: waves 0-3 hold the rows of the first, 4-7 those of the second, so
// every SIMD hosts one wave of each. Each wave keeps, for its whole key
// range:
//   * its Q rows as MFMA B operands in VGPRs,
//   * the fp32 output accumulator O^T (d x 32) in the MFMA C layout,
//   * the offset m and running sum l of its rows.
// Keys are streamed in tiles of 64 rows of K and V shared by all the
// workgroup's waves, loaded by the buffer loads' direct-to-LDS path into double-buffered
// LDS one step ahead of the block that reads them, with one barrier per
// step. A wave computes over the steps its rows reach and only loads and
// waits at the others; each wave sees every key tile of its rows, so no
// partial results are merged.
// fp32 io: 4 waves, 128 rows, one tile per step, loads through VGPRs.
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
// Online softmax in base 2 with c = |scale| * log2(e): P = 2^(c*S - m) with
// a row offset m that is raised lazily (see kSumMax below), alpha =
// 2^(m_old - m_new) rescales l and O when it is, and at the end O = O / l
// and LSE = ln2 * (m + log2 l). A negative scale is moved onto Q as an exact
// sign flip so that c > 0.
//
// Causal (top-left): query i sees key j iff j <= i. Key tiles past the last
// visible key of the workgroup are never loaded; a wave skips the tiles past
// its own last visible key, and only tiles that straddle the diagonal (or the
// end of the keys) evaluate the mask. Key rows at or beyond the sequence's
// key count read as zeros (a buffer bound, or a predicated load for fp32),
// so padding or a NaN-poisoned tail never reaches P.V (the FP8 d512 forward
// entry in the cudnn-frontend PR #554 merge log describes that failure:
// masking zeroes P, not V).
//
// Work order: blockIdx -> (query tile or causal tile pair, b*h), so all
// tiles of one (b, h) run on the same XCD when b*h is a multiple of 8 and
// share its L2.

#include <limits.h>
#include <math.h>

#include <atomic>
#include <type_traits>

#include "fwd_common.h"
#include "kernel_common.h"
#include "sdpa_internal.h"

namespace sdpa07 {
namespace {

// ---------------------------------------------------------------------------
// fp16 / bf16 io.
//
// Query tiles of 128 rows go in pairs of one (b|sequence, h), 32 rows per
// wave. Causal attention without a left bound pairs tiles (n-1-i, i): every
// pair holds the same causal work. Other masks pair adjacent tiles (2i,
// 2i+1), whose key ranges nearly coincide. A one-tile workgroup (4 waves;
// d = 64 and causal bands) runs one tile of a pair, and the grid places the
// pair's other tile on the same CU; the 8-wave workgroup (non-causal d = 128)
// runs both, waves 0-3 on tile A and 4-7 on tile B, so every SIMD hosts one
// wave of each, over one stream of key tiles that both start at key 0.
//
// Step s of the key loop loads one 64-key tile of K and V (each wave loads
// its share of it: a quarter or an eighth) and runs one straight-line block
// per wave whose rows see the tile (see `block`): the QK^T products of tile
// s+1, the P.V products of tile s-1 and the softmax of tile s, with the
// wave's share of the loads of later tiles spread over the block. A wave
// takes part in every step's barrier and loads, but computes only over the
// steps its own rows reach; when they end it drains its last P.V, and its
// rows leave after the last step. No partial results are merged: each wave
// sees every key tile of its rows.
//
// Softmax offsets are lazy: the offset m of a row (log2 units) changes only
// when a tile's scores rise well above it, and O and l always share it, so
// the result is exact whichever offsets are taken. Two ways of choosing it:
//  * checked after the fact (d = 64, where the softmax is the larger share
//    of a block's work): a block computes the P of its tile with the current
//    offset and the sum r of the rounded P over the lane's 32 scores, but no
//    row max. Right after the block, when every lane has r <= kSumMax (so
//    every P <= kSumMax, far inside the range of the 16-bit P) the sum joins
//    l; otherwise (scores well above the offset, an overflowed P, or a row
//    with no offset yet) the tile's scores, still in registers, give the new
//    offset m' = max(m, c * rowmax), O and l are rescaled by 2^(m - m') and
//    the tile's P is recomputed before the next block multiplies it into O.
//    A wave's first tile sets the offset from its own row max.
//  * decided before the block (d = 128, where the scores cannot stay live
//    through the block within the register budget): the previous block also
//    computes the row max of the next tile's scores, and the offset is raised
//    to it only when it exceeds the offset by more than kTau, so P <= 2^kTau;
//    the O rescale then runs after that block.
// The scale stays in fp32 (P = 2^(c*S - m), one fma per score): folding it
// into Q would round c*Q to the io type and shift scores by up to 2^-9 of
// their size.
constexpr float kSumMax = 4096.f;
// a compile-time ring phase (see the key loop's runs of four steps)
template <int N>
using kPh = std::integral_constant<int, N>;
constexpr float kTau = 8.f;

template <typename T, int D, bool CAUSAL, bool VARLEN>
__global__ void __launch_bounds__(fwd16_threads(D, CAUSAL))
    __attribute__((amdgpu_waves_per_eu(2, 2))) fwd16_kernel(FwdParams p) {
  constexpr int BM = kFwdBlockM, BN = kFwdBlockN;
  constexpr int NT = fwd16_threads(D, CAUSAL);
  constexpr int NW = NT / 64;          // waves: 4 (one query tile) or 8 (two)
  constexpr bool SPLIT = NW == 4;
  // K and V tiles go from memory straight into LDS (buffer loads with the
  // LDS flag): a wave's load instruction fills 1 KB of LDS, lane l writing
  // bytes [16l, 16l + 16). Rows are stored unpadded and each row's 16-byte
  // chunks are permuted by an XOR swizzle of the row index, so that the QK^T
  // operand reads (ds_read_b128, 16 rows per phase) and the transposing P.V
  // operand reads (ds_read_b64_tr_b16, 4 rows x 64 B per 32 lanes) hit
  // distinct banks; each lane loads the global chunk that its slot holds.
  // Tile u lives in buffer u mod NB of its ring (K or V). Step s reads K(s+1)
  // and V(s-1) and loads K(s+NB) and V(s+NB-2) into the buffers its
  // predecessor finished with, so every load has NB-1 steps to land before
  // the wait that needs it. At d = 64 a ring of four (80 KB of LDS with the
  // waves' Q rows) hides the latency of cold HBM reads; at d = 128 the LDS
  // holds two.
  constexpr int CH = D / 8;            // 16-byte chunks per row
  constexpr int RPI = 64 / CH;         // rows per load instruction
  constexpr int CPT = BN / RPI / (NT / 64);  // load instructions per wave per tensor per step
  static_assert(CPT >= 1 && BN % (RPI * (NT / 64)) == 0, "tile/workgroup mismatch");
  constexpr int NB = D <= 64 ? 4 : 2;
  constexpr int LK = NB - 1, LV = NB - 1;  // steps between a tile's load and its read
  // buffer of tile u >= -NB
  auto ring = [](int u) -> int { return (int)((unsigned)(u + NB) % (unsigned)NB); };
  constexpr int TILE = BN * D;         // elements per tile
  constexpr int QROWS = 32 * D;        // elements of one wave's Q rows
  // Q rows pass through LDS at d = 64 (whose epilogue reuses the area) and
  // in the 8-wave workgroup (whole rows per load instruction); the one-tile
  // d = 128 workgroup loads them straight into their registers, so that it
  // needs only the ring (64 KB) and two fit on a CU
  constexpr bool QLDS = D <= 64 || !SPLIT;
  constexpr int LDS_ELEMS = 2 * NB * TILE + (QLDS ? NW * QROWS : 0);
  using M = Mfma16<T>;
  using v8 = typename M::v8;
  __shared__ __attribute__((aligned(16))) T lds[LDS_ELEMS];
  T* const kbuf0 = lds;                 // [NB][TILE]
  T* const vbuf0 = lds + NB * TILE;     // [NB][TILE]
  // chunk permutation of row r (only r mod 16 matters)
  auto swz = [](int r) -> int {
    return D <= 64 ? (((r >> 1) ^ (((r >> 1) & 1) << 2)) & 7) : ((r ^ ((r & 3) << 2)) & 15);
  };

  // ---- work unit: two query tiles of one (b|sequence, h)
  // Dense: blockIdx -> (pair index, b*h). Packed: blockIdx -> (live pair of a
  // sequence, head), heads innermost, pairs of all sequences heaviest first
  // (the pair of a causal band without a left bound costs as many key blocks
  // as its longer tile: n_qt - j for pair j; other masks: the keys).
  const bool heavy_pair = CAUSAL && p.window_left < 0;
  // One tile per workgroup: the grid runs in rounds of 2R workgroups (R =
  // split_round, the compute-unit count); in a round, workgroup j < R takes
  // the first tile of the round's pair unit j and workgroup R + j its second,
  // the two that the dispatcher places on one CU when a full round is
  // resident (measured on MI355X: workgroups i and i + 256 of a 512-workgroup
  // grid at two per CU). The placement only matters for speed.
  int unit = blockIdx.x, half = 0;
  if constexpr (SPLIT) {
    const int n_units = gridDim.x / 2;
    const int R = p.split_round;
    const int r = blockIdx.x / (2 * R);
    const int rem = min(R, n_units - r * R);  // units in this round
    const int off = blockIdx.x - r * 2 * R;
    half = off / rem;
    unit = r * R + off % rem;
  }
  int pair, bi, hi;
  if constexpr (VARLEN) {
    hi = unit % p.h;
    const PackedUnit pu = packed_unit(unit / p.h, p.b, heavy_pair, [&](int s) -> int2 {
      const int lq = packed_len(p.cu_q, s, p.total_q);
      const int np = (lq + 2 * BM - 1) / (2 * BM);
      if (heavy_pair) return int2{np, (lq + BM - 1) / BM};
      return int2{np, max((packed_len(p.cu_kv, s, p.total_kv) + BN - 1) / BN, 1)};
    });
    if (pu.seq < 0) return;  // past the last pair (uniform over the workgroup)
    bi = pu.seq;
    pair = pu.j;
  } else {
    const int nbh = p.b * p.h;
    pair = unit / nbh;
    const int bh = unit % nbh;
    bi = bh / p.h;
    hi = bh % p.h;
  }
  const int hk = hi / (p.h / p.h_kv);  // K/V head of this query head
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
    k_off = (int64_t)k0 * p.k_ss + (int64_t)hk * p.k_sh;
    v_off = (int64_t)k0 * p.v_ss + (int64_t)hk * p.v_sh;
    lse_off = (int64_t)q0 * p.h + hi;
    lse_st = p.h;
  } else {
    q_len = p.s_q;
    kv_len = p.s_kv;
    q_off = (int64_t)bi * p.q_sb + (int64_t)hi * p.q_sh;
    o_off = (int64_t)bi * p.o_sb + (int64_t)hi * p.o_sh;
    k_off = (int64_t)bi * p.k_sb + (int64_t)hk * p.k_sh;
    v_off = (int64_t)bi * p.v_sb + (int64_t)hk * p.v_sh;
    lse_off = ((int64_t)bi * p.h + hi) * p.s_q;
    lse_st = 1;
  }
  // band of query row i: keys [i + shift - window, i + shift] (the upper
  // bound only when causal), within [0, kv_len)
  const int shift = p.bottom_right ? kv_len - q_len : 0;
  const int window = p.window_left < 0 ? (1 << 29) : p.window_left;
  const T* __restrict__ Q = (const T*)p.q + q_off;
  const T* __restrict__ K = (const T*)p.k + k_off;
  const T* __restrict__ V = (const T*)p.v + v_off;
  T* __restrict__ O = (T*)p.o + o_off;

  const int tid = threadIdx.x, lane = tid % 64;
  // wave-uniform values live in SGPRs so per-wave control flow stays scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int hf = lane / 32, col = lane % 32;

  // the two tiles: causal without a left bound pairs (n-1-i, i), others
  // (2i, 2i+1); a missing tile (odd count) is -1. Packed sequences pair the
  // tiles of each sequence among themselves (its own tile count n_qt).
  const int n_qt = VARLEN ? (q_len + BM - 1) / BM : p.n_qtiles;
  const int qt_p = heavy_pair ? n_qt - 1 - pair : 2 * pair;
  const int qt_q0 = heavy_pair ? pair : 2 * pair + 1;
  const int qt_q = (heavy_pair ? qt_q0 < qt_p : qt_q0 < n_qt) ? qt_q0 : -1;
  // the workgroup's tiles: A (waves 0-3) and B (waves 4-7), or with one tile
  // per workgroup A only
  const int qt_a = SPLIT && half ? qt_q : qt_p;
  const int qt_b = SPLIT ? -1 : qt_q;
  if (SPLIT && qt_a < 0) return;  // the pair has no second tile (uniform)
  // keys a tile's rows see: [lo, hi) (empty when the tile has no rows)
  auto tile_keys = [&](int qt, int& lo, int& hi2) {
    if (qt < 0 || qt * BM >= q_len) {
      lo = hi2 = 0;
      return;
    }
    const int last = min(q_len, (qt + 1) * BM) - 1;
    hi2 = CAUSAL ? min(kv_len, max(last + shift + 1, 0)) : kv_len;
    lo = min(hi2, max(qt * BM + shift - window, 0));
  };
  int a_lo, a_hi, b_lo, b_hi;
  tile_keys(qt_a, a_lo, a_hi);
  tile_keys(qt_b, b_lo, b_hi);
  // the workgroup's steps: tiles t0 .. t0 + n_steps - 1, one per step
  const bool a_any = a_hi > a_lo, b_any = b_hi > b_lo;
  const int kv_begin = !a_any ? b_lo : !b_any ? a_lo : min(a_lo, b_lo);
  const int kv_end = !a_any ? b_hi : !b_any ? a_hi : max(a_hi, b_hi);
  const int t0 = kv_begin / BN;
  const int n_steps = kv_end > kv_begin ? (kv_end + BN - 1) / BN - t0 : 0;

  const int qt = SPLIT || wave < 4 ? qt_a : qt_b;  // this wave's tile
  const int rg = wave % 4;                  // its row group
  const int row0 = qt * BM + rg * 32;       // first query row of this wave
  const int qi = row0 + col;                // this lane's query row
  const bool wave_active = qt >= 0 && row0 < q_len;
  const bool q_valid = wave_active && qi < q_len;
  // this wave's keys [wave_lo, wave_hi) and its steps [ws0, ws1)
  const int wave_last = min(row0 + 31, q_len - 1);
  const int wave_hi =
      !wave_active ? 0 : (CAUSAL ? min(kv_len, max(wave_last + shift + 1, 0)) : kv_len);
  const int wave_lo = min(wave_hi, max(row0 + shift - window, 0));
  int ws0 = 0, ws1 = 0;
  if (wave_hi > wave_lo) {
    ws0 = wave_lo / BN - t0;
    ws1 = (wave_hi + BN - 1) / BN - t0;
  }

  // s_waitcnt with only a vmcnt bound (gfx9 encoding: expcnt and lgkmcnt at
  // their maxima)
  auto wait_vm = [](auto n) {
    constexpr int N = decltype(n)::value;
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  };
  // Before the barrier of step s this wave's loads of K(s+1) and V(s-1) must
  // have landed: they were issued in steps s-LK and s-LV (V first, then K,
  // in each step), so the loads allowed to be outstanding are those issued
  // after the later of the two.
  constexpr int WAITN = CPT * (2 * LK - 2 < 2 * LV - 1 ? 2 * LK - 2 : 2 * LV - 1);
  using WaitStep = std::integral_constant<int, WAITN>;
  // the prologue's loads issued after K(0) before its wait: V(-1) and K(1)
  using WaitK0 = std::integral_constant<int, 2 * CPT>;
  using WaitAll = std::integral_constant<int, 0>;

  v8 qf[D / 16];
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  float l_run = 0.f;
  const float c = p.scale_log2;

  // K/V loads: each step the workgroup loads tile t0 + s through a buffer
  // resource rebased per tile whose byte bound ends with the last key row
  // any query of the workgroup sees (kv_end): rows past it read as zeros and
  // are masked anyway (rows are disjoint when the row stride is at least d,
  // which every dense layout satisfies; with overlapping rows the extra rows
  // are real, finite keys that the mask hides), with no per-lane test and no
  // memory touched past the keys; a tile outside the keys is all zeros.
  // Load instruction x of wave w covers rows RIT(x) .. RIT(x) + RPI - 1 of
  // the tile; lane l fills row RIT(x) + l / CH, slot l % CH.
  auto RIT = [&](int x) { return (NW * x + wave) * RPI; };
  const int drow = lane / CH;
  const int dchunk = (lane % CH) ^ swz(RIT(0) % 16 + drow);  // RIT(x) mod 16 is the same for all x
  static_assert((NW * RPI) % 16 == 0, "load rows change the swizzle phase");
  const int kvoff = drow * (int)p.k_ss * (int)sizeof(T) + dchunk * 16;
  const int vvoff = drow * (int)p.v_ss * (int)sizeof(T) + dchunk * 16;
  // buffer resource of key tile t0 + t (zero bytes for tiles outside the
  // keys), from the tile's first row tb; built in scalar code outside the
  // fused blocks
  const T* __restrict__ K0 = K + (int64_t)t0 * BN * p.k_ss;
  const T* __restrict__ V0 = V + (int64_t)t0 * BN * p.v_ss;
  const int kv_rel = kv_end - t0 * BN;  // keys from tile t0 on
  // tiles 0 .. n_full-1 (from t0) hold BN keys, tile n_full the remaining
  // kv_rel mod BN (if any), later tiles none
  const int n_full = kv_rel / BN, edge_rows = kv_rel % BN;
  auto tile_bytes = [&](int64_t stride, int rows) -> int {
    return rows <= 0 ? 0 : ((rows - 1) * (int)stride + D) * (int)sizeof(T);
  };
  const int full_k = tile_bytes(p.k_ss, BN), edge_k = tile_bytes(p.k_ss, edge_rows);
  const int full_v = tile_bytes(p.v_ss, BN), edge_v = tile_bytes(p.v_ss, edge_rows);
  static_assert(LK == LV, "one load group per step: V(s-1+LV), then K(s+1+LK)");
  const int s_edge = n_full - 1 - LK;  // first step whose K tile is not a whole one
  auto tile_bytes_at = [&](int t, int full, int edge) -> int {
    return (t < 0 || t > n_full) ? 0 : t < n_full ? full : edge;
  };
  auto make_rsrc = [&](const T* __restrict__ tb, int bytes) -> i32x4 {
    const unsigned long long a = (unsigned long long)tb;
    return i32x4{(int)(unsigned)a, (int)((unsigned)(a >> 32) & 0xffffu), bytes, kBufferFlags};
  };
  auto tile_rsrc_at = [&](const T* __restrict__ tb, int t, int full, int edge) -> i32x4 {
    return make_rsrc(tb, tile_bytes_at(t, full, edge));
  };
  // LDS byte address of the array's element e (the M0 operand of the
  // direct-to-LDS loads), from the array's own LDS address
  const unsigned lds_a = (unsigned)(size_t)(__attribute__((address_space(3))) T*)lds;
  auto lds_at = [&](int e) -> unsigned { return lds_a + (unsigned)e * (unsigned)sizeof(T); };
  auto dma = [&](i32x4 rs, int voff, int soff, unsigned dst) { lds_dma16(rs, voff, soff, dst); };
  // this wave's load instruction x of tile u's K (V) into its buffer (u >= -1;
  // tile -1 is all zeros)
  // (the buffer index: ring(u) for tile u >= -1)
  auto kdma = [&](i32x4 r, int buf, int x) {
    dma(r, kvoff, RIT(x) * (int)p.k_ss * (int)sizeof(T), lds_at(buf * TILE + RIT(x) * D));
  };
  auto vdma = [&](i32x4 r, int buf, int x) {
    dma(r, vvoff, RIT(x) * (int)p.v_ss * (int)sizeof(T), lds_at((NB + buf) * TILE + RIT(x) * D));
  };
  auto rsrc_k = [&](int u) -> i32x4 {
    return tile_rsrc_at(K0 + (int64_t)u * BN * p.k_ss, u, full_k, edge_k);
  };
  auto rsrc_v = [&](int u) -> i32x4 {
    return tile_rsrc_at(V0 + (int64_t)u * BN * p.v_ss, u, full_v, edge_v);
  };
  // first rows of the tiles the next step's loads fill (K of step s+1+LK,
  // V of step s-1+LV), advanced by one tile of rows per step so that the
  // loop carries plain pointer increments
  const T* kstep_ptr = K0 + (int64_t)(1 + LK) * BN * p.k_ss;
  const T* vstep_ptr = V0 + (int64_t)(LV - 1) * BN * p.v_ss;

  // Softmax state (per lane = per query row; both halves agree):
  //   m_cur  offset (log2 units) of l, of O and of the P that the next block
  //          computes (-inf while the row has seen no score); with decided
  //          offsets l and O take it only once that block has run
  //   a_cur  (decided offsets) factor for l (in the block) and for O (after
  //          it) when the offset was raised before the block, else 1
  //   mx_nxt (decided offsets) row max of the raw scores the last block
  //          produced
  constexpr bool CHECK_AFTER = D <= 64;
  float m_cur = -INFINITY, a_cur = 1.f, mx_nxt = -INFINITY;
  // kept with m_cur: the offset a block subtracts (0 for a row without one)
  // and the wave's rows without one (a scalar lane mask)
  float m_off_cur = 0.f;
  unsigned long long no_off = __builtin_amdgcn_ballot_w64(true);
  auto set_m = [&](float m) {
    m_cur = m;
    m_off_cur = m == -INFINITY ? 0.f : m;
    no_off = __builtin_amdgcn_ballot_w64(m == -INFINITY);
  };
  constexpr int NPAIR = 16;  // 32 scores per lane, in pairs
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
  // P of score pair pp (keys 2pp, 2pp+1 of the lane's 32, in the order of
  // the P.V B operands) with offset m_off, rounded to the io type and packed
  auto p_pair = [&](const f32x16(&sv)[2], int pp, float m_off) {
    const int t = pp / 4, e2 = pp % 4;
    const float s0 = sv[t / 2][8 * (t % 2) + 2 * e2];
    const float s1 = sv[t / 2][8 * (t % 2) + 2 * e2 + 1];
    const f32x2 x = {fast_exp2(fmaf(s0, c, -m_off)), fast_exp2(fmaf(s1, c, -m_off))};
    return __builtin_convertvector(x, typename Pack2<T>::type);
  };
  // Settling the P that a block just computed, before the next block
  // multiplies it into O (sv: the tile's masked scores, pv: its P, r: the
  // lane's sum of it). p_ok: every lane's sum is within kSumMax and the row
  // had an offset, so r joins l. Otherwise fix raises the offset to the
  // tile's row max, rescales O and l and recomputes the tile's P.
  auto p_ok = [&](float r) -> bool {
    return (__builtin_amdgcn_ballot_w64(r > kSumMax) | no_off) == 0;
  };
  auto fix = [&](const f32x16(&sv)[2], v8(&pv)[4]) {
    const float m_new = fmaxf(m_cur, row_max(sv) * c);
    const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_cur - m_new);
    const float m_off = m_new == -INFINITY ? 0.f : m_new;
    // P and O are rewritten in place, pair by pair (operands tied to their
    // own registers, no temporaries)
    float r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      i32x4 w = __builtin_bit_cast(i32x4, pv[t]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const auto h = p_pair(sv, 4 * t + e, m_off);
        if (e & 1) r1 = dot2_ones<T>(h, r1);
        else r0 = dot2_ones<T>(h, r0);
        int o = w[e];
        asm volatile("v_mov_b32 %0, %1" : "+v"(o) : "v"(__builtin_bit_cast(int, h)));
        w[e] = o;
      }
      pv[t] = __builtin_bit_cast(v8, w);
    }
    l_run = l_run * alpha + (r0 + r1);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x = acc[db][e];
        asm volatile("v_mul_f32 %0, %0, %1" : "+v"(x) : "v"(alpha));
        acc[db][e] = x;
      }
    set_m(m_new);
  };
  auto settle = [&](const f32x16(&sv)[2], v8(&pv)[4], float r) {
    if (__builtin_expect(p_ok(r), 1)) l_run += r;
    else fix(sv, pv);
  };
  // Decided offsets: the decision for the coming block's scores, given their
  // raw row max mx. Returns true (wave-uniform) when some row raised its
  // offset; then a_cur holds 2^(m_old - m_new) for those rows (1 elsewhere).
  auto decide = [&](float mx) -> bool {
    const float mt = mx * c;  // log2 units
    const bool need = m_cur == -INFINITY ? mt != -INFINITY : mt > m_cur + kTau;
    a_cur = 1.f;
    if (!__any(need)) return false;
    const float m_new = need ? mt : m_cur;
    a_cur = need ? fast_exp2(m_cur - m_new) : 1.f;  // 0 for a row's first offset
    set_m(m_new);
    return true;
  };

  // One pipeline block of step s, straight-line code:
  //   QK  : S_next = K_next Q^T                  (MFMAs 0 .. NQK-1)
  //   PV  : O^T += V_prev^T P_prev^T             (MFMAs NQK .. NM-1)
  //   SM  : P_cur = 2^(c S_cur - m), its sum     (VALU, early chunks)
  //   MX  : (decided offsets) row max of S_next  (VALU, last chunks, once
  //                                               the QK results are complete)
  //   MEM : this wave's direct-to-LDS loads of V(s-1+LV) and K(s+1+LK),
  //         one instruction per chunk
  // It is emitted as NM chunks, each = the LDS read for the MFMA PF chunks
  // ahead, one MFMA, a slice of the VALU work and at most one load; the
  // slices are pinned to their chunk so the VALU work issues while the MFMA
  // pipe is busy.
  constexpr int NQK = 2 * (D / 16);
  constexpr int NPV = 4 * (D / 32);
  constexpr int NM = NQK + NPV;
  constexpr int PF = D <= 64 ? 3 : 2;                     // LDS read-ahead (chunks)
  constexpr int EXP_SPAN = CHECK_AFTER ? NM - 2 : NM - 6;
  constexpr int EXP_CHUNKS = EXP_SPAN < 16 ? EXP_SPAN : 16;  // chunks holding the exps
  constexpr int MX0 = NM - 4;  // (decided offsets) chunks MX0 .. MX0+2: max of S_next
  constexpr int MEM0 = 1;                                 // chunks MEM0 .. MEM0+2*CPT-1
  static_assert(MEM0 + 2 * CPT <= NM, "not enough chunks for the memory ops");
  const int vrow = 4 * hf + (lane % 16) / 4;
  const int vcol = 16 * ((lane / 16) % 2) + 4 * (lane % 4);
  // MFMA A operands: K rows 32mb + col, d 16ks + 8hf .. +7 (S^T = K Q^T), and
  // V^T rows (d) 32db + col for keys 16t + 8(e/4) + 4hf + e%4 (O^T = V^T P^T).
  // Element offsets within a tile carry the chunk swizzle (rows 32mb + col
  // and 16t + r share the swizzle of col and r); they are loop-invariant
  // (no per-lane arrays: an indexed private array could be moved to LDS).
  const int sk = swz(col % 16), sv0 = swz(vrow), sv1 = swz(vrow + 8);
  auto read_k = [&](const T* kb, int ks, int mb) -> v8 {
    return *(const v8*)&kb[(32 * mb + col) * D + (((2 * ks + hf) ^ sk) * 8)];
  };
  auto read_v = [&](const T* vb, int t, int db) -> v8 {
    const int c = 4 * db + vcol / 8;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(vb + (16 * t + vrow) * D + ((c ^ sv0) * 8) +
                                                   vcol % 8));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(vb + (16 * t + vrow + 8) * D +
                                                   ((c ^ sv1) * 8) + vcol % 8));
    return __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // S of a wave's first tile alone (its P.V and softmax have nothing to do)
  auto qk_only = [&](const T* kb, f32x16(&s_out)[2]) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        s_out[mb] = M::mma(read_k(kb, ks, mb), qf[ks], ks == 0 ? f32x16{} : s_out[mb]);
    if constexpr (!CHECK_AFTER) mx_nxt = row_max(s_out);
  };
  // a wave's last P.V alone (after its last step)
  auto pv_only = [&](const T* vb, const v8(&p_last)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] = M::mma(read_v(vb, t, db), p_last[t], acc[db]);
  };
  // Buffers of step s: K(s+1) and V(s-1) are read, V(s-1+LV) and K(s+1+LK)
  // written. With a ring of two all four are rbuf = (s + 1) mod 2 or its
  // other one, passed in so that a loop over pairs of steps keeps the LDS
  // operand addresses of both steps loop-invariant; a deeper ring adds a
  // scalar buffer offset per step to the invariant lane addresses.
  // (ph: the step's ring phase s mod 4 when known at compile time, which
  // turns the ring buffers' offsets into constants; -1: computed from s)
  auto block = [&](auto ph, int s, int rbuf, const f32x16(&s_cur)[2], f32x16(&s_nxt)[2],
                   const v8(&p_prev)[4],
                   v8(&p_cur)[4], const i32x4& rk, const i32x4& rv) -> float {
    constexpr int PH = decltype(ph)::value;
    constexpr bool STATIC = PH >= 0 && NB == 4;
    const int kr = NB == 2 ? rbuf : STATIC ? (PH + 1) & 3 : ring(s + 1);
    const int vr = NB == 2 ? rbuf : STATIC ? (PH + 3) & 3 : ring(s - 1);
    const int kw = NB == 2 ? rbuf ^ 1 : STATIC ? PH : ring(s + 1 + LK);
    const int vw = NB == 2 ? rbuf ^ 1 : STATIC ? (PH + 2) & 3 : ring(s - 1 + LV);
    const T* kb = kbuf0 + kr * TILE;  // K of step s+1
    const T* vb = vbuf0 + vr * TILE;  // V of step s-1
    auto read_op = [&](int i) -> v8 {
      if (i < NQK) return read_k(kb, i / 2, i % 2);
      return read_v(vb, (i - NQK) / (D / 32), (i - NQK) % (D / 32));
    };
    auto mem = [&](int i) {  // loads of V(s-1+LV), then K(s+1+LK)
      const int k = i - MEM0;
      if (k < 0 || k >= 2 * CPT) return;
      if (k < CPT) vdma(rv, vw, k);
      else kdma(rk, kw, k - CPT);
    };
    const float m_off = m_off_cur;
    float r0 = 0.f, r1 = 0.f, mxa = -INFINITY, mxb = -INFINITY;
    i32x4 pk[4];
    auto slice = [&](int i) {
      if (i < EXP_CHUNKS) {
        const int p0 = i * NPAIR / EXP_CHUNKS, p1 = (i + 1) * NPAIR / EXP_CHUNKS;
#pragma unroll
        for (int pp = p0; pp < p1; ++pp) {
          const auto h = p_pair(s_cur, pp, m_off);
          const int hb = __builtin_bit_cast(int, h);
          pin(hb);
          pk[pp / 4][pp % 4] = hb;
          if (pp & 1) r1 = dot2_ones<T>(h, r1);
          else r0 = dot2_ones<T>(h, r0);
        }
      }
      if constexpr (CHECK_AFTER) {
        if (i == EXP_CHUNKS) pin(r0), pin(r1);
      } else {
        if (i == EXP_CHUNKS) {
          l_run = l_run * a_cur + (r0 + r1);
          pin(l_run);
        }
        if (i == MX0) {
          mxa = fmaxf(fmaxf(s_nxt[0][0], s_nxt[0][1]), s_nxt[0][2]);
          mxb = fmaxf(fmaxf(s_nxt[0][3], s_nxt[0][4]), s_nxt[0][5]);
#pragma unroll
          for (int r = 6; r < 14; r += 4) {
            mxa = fmaxf(fmaxf(mxa, s_nxt[0][r]), s_nxt[0][r + 1]);
            mxb = fmaxf(fmaxf(mxb, s_nxt[0][r + 2]), s_nxt[0][r + 3]);
          }
          mxa = fmaxf(fmaxf(mxa, s_nxt[0][14]), s_nxt[0][15]);
          pin(mxa);
          pin(mxb);
        }
        if (i == MX0 + 1) {
#pragma unroll
          for (int r = 0; r < 16; r += 4) {
            mxa = fmaxf(fmaxf(mxa, s_nxt[1][r]), s_nxt[1][r + 1]);
            mxb = fmaxf(fmaxf(mxb, s_nxt[1][r + 2]), s_nxt[1][r + 3]);
          }
          pin(mxa);
          pin(mxb);
        }
        if (i == MX0 + 2) {
          const float mx = fmaxf(mxa, mxb);
          mx_nxt = fmaxf(mx, other_half(mx));
          pin(mx_nxt);
        }
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
      mem(i);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) p_cur[t] = __builtin_bit_cast(v8, pk[t]);
    return r0 + r1;
  };

  // The start of step s, common to every wave: the descriptors of the tiles
  // this step's loads fill, the wait for this wave's loads of the tiles the
  // step reads, and one barrier (every wave's loads have then landed, and
  // every wave is done with the buffers this step's loads overwrite).
  auto step_begin = [&](int s, i32x4& rk, i32x4& rv) {
    // both tiles whole unless the later one (K, tile s + 1 + LK) reaches the
    // keys' edge tile (the V tile, s - 1 + LV >= 0, is never before the first)
    const int tk = s + 1 + LK, tv = s - 1 + LV;
    int bk = full_k, bv = full_v;
    if (__builtin_expect(s >= s_edge, 0)) {
      bk = tile_bytes_at(tk, full_k, edge_k);
      bv = tile_bytes_at(tv, full_v, edge_v);
    }
    rk = make_rsrc(kstep_ptr, bk);
    rv = make_rsrc(vstep_ptr, bv);
    kstep_ptr += BN * p.k_ss;
    vstep_ptr += BN * p.v_ss;
    wait_vm(WaitStep{});
    __builtin_amdgcn_s_barrier();
  };
  // No band bound cuts the tile with first key kbase iff kbase lies in
  // [uncut_lo, uncut_hi]: the left bound cuts it when kbase < uncut_lo, the
  // causal bound when kbase > row0 + shift - BN + 1, the end of the keys when
  // kbase > kv_len - BN. One unsigned compare per step tests the interval
  // (an empty interval makes every tile cut: kbase >= 0 > INT_MIN).
  int uncut_lo = wave_last + shift - window;
  int uncut_hi = kv_len - BN;
  if (CAUSAL) uncut_hi = min(uncut_hi, row0 + shift - BN + 1);
  unsigned uncut_span = (unsigned)uncut_hi - (unsigned)uncut_lo;
  if (uncut_hi < uncut_lo) {
    uncut_lo = INT_MIN;
    uncut_span = 0u;
  }
  // A step without a block: the wave's share of the step's loads only.
  auto light_step = [&](int s) {
    i32x4 rk, rv;
    step_begin(s, rk, rv);
#pragma unroll
    for (int x = 0; x < CPT; ++x) vdma(rv, ring(s - 1 + LV), x);
#pragma unroll
    for (int x = 0; x < CPT; ++x) kdma(rk, ring(s + 1 + LK), x);
  };
  // Step s with a block: the mask of this tile's scores where a band bound
  // cuts it, then the fused block; with checked offsets it returns the
  // lane's sum of the P it computed, for the caller to settle (with decided
  // offsets the decision comes before the block and the O rescale after it). Every block runs the
  // same code; the first block's P.V is neutralised by
  // data (P_prev = 0), and the last block's QK of the next tile computes a
  // value that is never used.
  // (FIRST: the wave's first tile, a separate instantiation so that the row
  // max it takes, and the canonicalisation of the masked scores that it
  // needs, stay out of the other steps)
  auto step = [&](auto first, auto ph, int s, int rbuf, f32x16(&s_cur)[2], f32x16(&s_nxt)[2],
                  const v8(&p_prev)[4], v8(&p_cur)[4]) -> float {
    constexpr bool FIRST = decltype(first)::value;
    i32x4 rk, rv;
    step_begin(s, rk, rv);
    const int kbase = (t0 + s) * BN;  // this step's key tile
    const bool any_cut = (unsigned)kbase - (unsigned)uncut_lo > uncut_span;
    const bool cut_causal = CAUSAL && kbase + BN - 1 > row0 + shift;
    const bool cut_left = kbase < wave_last + shift - window;
    const bool cut_end = kbase + BN > kv_len;
    if constexpr (CHECK_AFTER) {
      if (any_cut)
        mask_tile<CAUSAL>(s_cur, kbase, qi, kv_len, hf, shift, window, cut_causal, cut_left,
                          cut_end);
      if constexpr (FIRST) set_m(row_max(s_cur) * c);  // the first tile's own row max
      return block(ph, s, rbuf, s_cur, s_nxt, p_prev, p_cur, rk, rv);  // P_cur still to settle
    } else {
      float mx = mx_nxt;
      if (any_cut) {
        mask_tile<CAUSAL>(s_cur, kbase, qi, kv_len, hf, shift, window, cut_causal, cut_left,
                          cut_end);
        mx = row_max(s_cur);
      }
      const bool rescale = decide(mx);
      const float a_blk = a_cur;
      block(ph, s, rbuf, s_cur, s_nxt, p_prev, p_cur, rk, rv);
      if (rescale) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] *= a_blk;
      }
      return 0.f;
    }
  };

  // Epilogue of a wave: combine the two lane halves' partial sums, normalise,
  // and store its rows and the statistic. A lane holds 4-d pieces of its
  // row's output spread over the row (the C layout of O^T); written straight
  // out, every store instruction touches 32 rows with 16 bytes each. At
  // d = 64 the rows go through the wave's own Q area instead (its Q is in
  // registers by then): the lanes write their pieces into rows laid out
  // [row][d], with the row's 16-byte chunks XOR-permuted by the row index so
  // that the 32 rows of a write spread over the banks, then read back whole
  // chunks, so that each store instruction writes 8 complete rows. (At
  // d = 128 the kernel has no registers to spare for the exchange and keeps
  // the direct stores.)
  // where a wave stages its finished rows: its Q area (d = 64, and the
  // 8-wave workgroup), else its quarter of the K ring, which no wave reads
  // after the last step's barrier
  T* const qbuf = lds + (QLDS ? 2 * NB * TILE + wave * QROWS : wave * QROWS);
  static_assert(QLDS || NW * QROWS <= NB * TILE, "staging rows exceed the K ring");
  // The epilogue in two parts: epi_stage normalises the rows into the
  // staging area and keeps the lane's statistic; epi_store reads the rows
  // back and stores them whole, with the statistic. At d = 64 rows finished
  // in the middle of the key loop are stored only after its last step: a
  // global store counts in vmcnt like the loads, so a store in flight would
  // hold up the wave's next counted wait (and through the barrier the
  // workgroup) until memory has acknowledged it. At d = 128 a wave that
  // finishes early keeps its rows in the accumulator (its last P.V done at
  // once) and stages them only after the last barrier, since the one-tile
  // workgroup stages in its K ring, in use until then.
  int st_row0 = 0;          // the staged rows: first row, any row, and the
  bool st_active = false;   // lane's row and statistic
  bool st_qvalid = false;
  float st_lse = 0.f;
  auto epi_stage = [&](auto staged) {
    constexpr bool STAGED = decltype(staged)::value;
    const float l_tot = l_run + other_half(l_run);
    // (the hardware reciprocal: within an ulp, far below the io type's
    // rounding of O)
    const float inv = l_tot > 0.f ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
    typedef T t4 __attribute__((ext_vector_type(4)));
    st_row0 = row0;
    st_active = wave_active;
    st_qvalid = q_valid;
    st_lse = l_tot > 0.f ? (m_cur + __log2f(l_tot)) * kLn2 : -INFINITY;
    if constexpr (STAGED) {
      constexpr int CPR = D / 8;  // 16-byte chunks per row
      // (the lane's offsets from a fresh copy of its index, so that each
      // inlined copy computes them where it runs instead of sharing ones
      // computed early and held in registers)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int cl = ln % 32, hl = ln / 32;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          t4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = (T)(acc[db][4 * rq + e] * inv);
          *(t4*)&qbuf[cl * D + ((4 * db + rq) ^ (cl % CPR)) * 8 + 4 * hl] = ov;
        }
    } else {
      // (the output and statistic bases pass an empty asm for the same
      // reason)
      T* Ob = fresh_uniform(O);
      float* lse_b = fresh_uniform(p.lse + lse_off);
      if (q_valid) {
        T* orow = Ob + (int64_t)qi * p.o_ss;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            t4 ov;
#pragma unroll
            for (int e = 0; e < 4; ++e) ov[e] = (T)(acc[db][4 * rq + e] * inv);
            *(t4*)(orow + 32 * db + 8 * rq + 4 * hf) = ov;
          }
        if (hf == 0 && p.lse) lse_b[(int64_t)qi * lse_st] = st_lse;
      }
    }
  };
  auto epi_store = [&]() {
    {
      constexpr int CPR = D / 8;     // 16-byte chunks per row
      constexpr int RPS = 64 / CPR;  // rows per store instruction
      T* Ob = fresh_uniform(O);
      float* lse_b = fresh_uniform(p.lse + lse_off);
      int ln = lane;
      asm volatile("" : "+v"(ln));
      // the wave reads back what its other lanes wrote: LDS operations of
      // one wave complete in order; the fences keep the compiler's order and
      // wait
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int sr = ln / CPR, sc = ln % CPR;
      // all of the lane's chunks first, so that the stores wait once (at
      // d = 64 row groups are RPS rows apart and share the chunk permutation)
      i32x4 vrow[32 / RPS];
      if constexpr (RPS % CPR == 0) {
        const int cofs = sr * D + (sc ^ (sr % CPR)) * 8;
#pragma unroll
        for (int x = 0; x < 32 / RPS; ++x) vrow[x] = *(const i32x4*)&qbuf[x * RPS * D + cofs];
      } else {
#pragma unroll
        for (int x = 0; x < 32 / RPS; ++x) {
          const int r = x * RPS + sr;
          vrow[x] = *(const i32x4*)&qbuf[r * D + (sc ^ (r % CPR)) * 8];
        }
      }
      // the stores carry the system-scope cache policy (sc0 sc1), which
      // writes the rows through to memory as they are stored; measured
      // faster than leaving them dirty in the L2 for the kernel's end. They
      // are buffer stores over the RPS rows of each instruction, whose
      // per-lane offsets fit 31 bits unless a row stride is beyond 2^26
      // elements (then plain stores); a wave whose 32 rows all exist, with
      // a row stride below 2^24 elements, stores through one descriptor at
      // its first row and a scalar offset per row group.
      const bool wt = p.o_ss < (1 << 26);
      if (st_active && st_row0 + 32 <= q_len && p.o_ss < (1 << 24)) {
        const T* base = Ob + (int64_t)max(st_row0, 0) * p.o_ss;
        const auto rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7fffffff, kBufferFlags);
        const int voff = (sr * (int)p.o_ss + sc * 8) * (int)sizeof(T);
#pragma unroll
        for (int x = 0; x < 32 / RPS; ++x)
          __builtin_amdgcn_raw_buffer_store_b128(vrow[x], rs, voff,
                                                 x * RPS * (int)p.o_ss * (int)sizeof(T),
                                                 kCacheSystemScope);
      } else {
#pragma unroll
        for (int x = 0; x < 32 / RPS; ++x) {
          const int r = x * RPS + sr;
          if (st_active && st_row0 + r < q_len) {
            if (wt) {
              const T* base = Ob + (int64_t)max(st_row0 + x * RPS, 0) * p.o_ss;
              __builtin_amdgcn_raw_buffer_store_b128(
                  vrow[x],
                  __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7fffffff, kBufferFlags),
                  (sr * (int)p.o_ss + sc * 8) * (int)sizeof(T), 0, kCacheSystemScope);
            } else {
              *(i32x4*)(Ob + (int64_t)(st_row0 + r) * p.o_ss + sc * 8) = vrow[x];
            }
          }
        }
      }
      if (st_qvalid && hf == 0 && p.lse) lse_b[(int64_t)(st_row0 + col) * lse_st] = st_lse;
    }
  };
  auto epilogue = [&]() {
    if constexpr (D <= 64) {
      epi_stage(std::true_type{});
      epi_store();
    } else {
      epi_stage(std::false_type{});
    }
  };

  if (n_steps == 0) {
    epilogue();  // no key anywhere: O = 0, LSE = -inf
    return;
  }

  // Prologue: this wave's 32 query rows into its own LDS area (rows past the
  // sequence read as zeros), then the loads that steps -(LK+1) .. -1 would
  // have issued, in the steps' order (V(b-1+LV) when it is a step >= -1, then
  // K(b+1+LK)): K(0 .. LK) and V(-1 .. LV-2) (V(-1), read by a first block's
  // no-op P.V, is all zeros). Only Q and K(0) have to land before the first
  // block; the steps' own waits cover the rest.
  i32x4 qraw[D / 16];  // (Q straight to registers) the lane's chunks as loaded
  {
    const int rows = wave_active ? min(q_len - row0, 32) : 0;
    const T* qb = Q + (int64_t)max(row0, 0) * p.q_ss;
    const int bytes = rows <= 0 ? 0 : ((rows - 1) * (int)p.q_ss + D) * (int)sizeof(T);
    if constexpr (QLDS) {
      const unsigned long long a = (unsigned long long)qb;
      const i32x4 rq = {(int)(unsigned)a, (int)((unsigned)(a >> 32) & 0xffffu), bytes,
                        kBufferFlags};
      // instruction x fills rows x * RPI + lane / CH of the wave's 32, each
      // lane the global chunk that its slot holds under that row's swizzle
#pragma unroll
      for (int x = 0; x < 32 / RPI; ++x) {
        const int qdchunk = (lane % CH) ^ swz((x * RPI + drow) % 16);
        const int qvoff = drow * (int)p.q_ss * (int)sizeof(T) + qdchunk * 16;
        dma(rq, qvoff, x * RPI * (int)p.q_ss * (int)sizeof(T),
            lds_at(2 * NB * TILE + wave * QROWS + x * RPI * D));
      }
    } else {
      // lane: row col, chunks 2ks + hf (the B-operand layout below)
      const auto rq = __builtin_amdgcn_make_buffer_rsrc((void*)qb, (short)0, bytes, kBufferFlags);
      const int qvoff = col * (int)p.q_ss * (int)sizeof(T) + hf * 16;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        qraw[ks] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, qvoff, 32 * ks, 0));
    }
  }
  // the loads step b would have issued: V(b-1+LV) when it is a tile >= -1,
  // then K(b+1+LK)
  auto prologue_loads = [&](int b) {
    if (b - 1 + LV >= -1) {
      const i32x4 r = rsrc_v(b - 1 + LV);
#pragma unroll
      for (int x = 0; x < CPT; ++x) vdma(r, ring(b - 1 + LV), x);
    }
    const i32x4 r = rsrc_k(b + 1 + LK);
#pragma unroll
    for (int x = 0; x < CPT; ++x) kdma(r, ring(b + 1 + LK), x);
  };
  // Q, K(0) and the first block's V(-1), K(1) go first; the rest of the
  // ring (needed from step 1 on) is issued after Q and K(0) have landed, so
  // that with cold caches it does not compete with them for HBM. The issue
  // order is that of the steps either way, which the counted waits rely on.
  constexpr int B_LATE = -(LK + 1) + 2;  // first step whose loads wait
  static_assert(LV == LK, "one load group per step");
#pragma unroll
  for (int b = -(LK + 1); b < (B_LATE < 0 ? B_LATE : 0); ++b) prologue_loads(b);
  f32x16 sa[2], sb[2];
  v8 pa[4], pb[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    pa[t] = v8{};
    pb[t] = v8{};
  }
  wait_vm(WaitK0{});  // this wave's loads of Q and K(0); then every wave's
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int b = B_LATE; b < 0; ++b) prologue_loads(b);
  // Q rows as B operands of S^T = K Q^T: lane holds Q[qi][16ks + 8hf .. +7]
  // (a negative scale is moved onto Q exactly: its sign bits flipped by a
  // wave-uniform mask)
  const int qsign = __builtin_amdgcn_readfirstlane(p.negate_q ? (int)0x80008000 : 0);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    i32x4 raw;
    if constexpr (QLDS) raw = *(const i32x4*)&lds[2 * NB * TILE + wave * QROWS + col * D +
                                                   (((2 * ks + hf) ^ sk) * 8)];
    else raw = qraw[ks];
    raw ^= qsign;
    qf[ks] = __builtin_bit_cast(v8, raw);
  }
  if (ws1 > ws0 && ws0 == 0) qk_only(kbuf0, sa);  // S of step 0 (K(0) is in buffer 0)

  int s = 0;
  // steps before this wave's first tile; the last of them computes S of
  // that tile (K(ws0) has landed at its barrier)
  for (; s < ws0; ++s) {
    light_step(s);
    if (s == ws0 - 1) qk_only(kbuf0 + ring(ws0) * TILE, sa);
  }
  // this wave's steps: even offsets from ws0 use S_cur = sa, S_next = sb,
  // P_prev = pb, P_cur = pa; odd ones the other way round
  using kFirst = std::true_type;
  using kNext = std::false_type;
  using kDyn = std::integral_constant<int, -1>;
  bool last_in_pa = true;
  if (ws1 > ws0) {
    if constexpr (CHECK_AFTER) {
      // the first step on its own, then pairs from an odd offset. A tile
      // whose P needs a new offset leaves the inner loop and is fixed
      // outside it (with the rest of its pair), so that the loop's code
      // holds no O rescale: one inside it made the register allocator move
      // O and P between two register sets, with a copy of both every step.
      settle(sa, pa, step(kFirst{}, kDyn{}, s, (s + 1) & 1, sa, sb, pb, pa));
      ++s;
      // Pairs from odd offsets. With a ring of four and ws0 even, a pair
      // that starts at a step s = 1 mod 4 begins a run of four steps whose
      // ring phases 1, 2, 3, 0 are compile-time constants; other pairs
      // (to reach that alignment, the last two or three steps, after an
      // offset fix) compute their buffers from s.
      const bool quads = NB == 4 && (ws0 & 1) == 0;
      while (s + 1 < ws1) {
        int ev = 0;  // 1: the pair's first tile needs fixing, 2: its second
        const int ba = (s + 1) & 1;  // the pairs' first steps read buffer ba
        if (quads && (s & 3) == 1) {
          for (; s + 3 < ws1; s += 4) {
            const float r1 = step(kNext{}, kPh<1>{}, s, ba, sb, sa, pa, pb);
            if (__builtin_expect(!p_ok(r1), 0)) {
              ev = 1;
              break;
            }
            l_run += r1;
            const float r2 = step(kNext{}, kPh<2>{}, s + 1, ba ^ 1, sa, sb, pb, pa);
            if (__builtin_expect(!p_ok(r2), 0)) {
              ev = 2;
              break;
            }
            l_run += r2;
            const float r3 = step(kNext{}, kPh<3>{}, s + 2, ba, sb, sa, pa, pb);
            if (__builtin_expect(!p_ok(r3), 0)) {
              ev = 3;
              break;
            }
            l_run += r3;
            const float r4 = step(kNext{}, kPh<0>{}, s + 3, ba ^ 1, sa, sb, pb, pa);
            if (__builtin_expect(!p_ok(r4), 0)) {
              ev = 4;
              break;
            }
            l_run += r4;
          }
          if (ev > 2) {  // in the run's second pair
            s += 2;
            ev -= 2;
          }
        }
        if (ev == 0) {
          if (s + 1 >= ws1) break;
          const float ra = step(kNext{}, kDyn{}, s, ba, sb, sa, pa, pb);
          if (__builtin_expect(!p_ok(ra), 0)) {
            ev = 1;
          } else {
            l_run += ra;
            const float rb = step(kNext{}, kDyn{}, s + 1, ba ^ 1, sa, sb, pb, pa);
            if (__builtin_expect(!p_ok(rb), 0)) ev = 2;
            else l_run += rb;
          }
          if (ev == 0) {
            s += 2;
            continue;
          }
        }
        if (ev == 1) {
          fix(sb, pb);  // tile s: scores in sb, P in pb
          settle(sa, pa, step(kNext{}, kDyn{}, s + 1, (s + 2) & 1, sa, sb, pb, pa));
        } else {
          fix(sa, pa);  // tile s + 1: scores in sa, P in pa
        }
        s += 2;
      }
      last_in_pa = s >= ws1;
      if (s < ws1) {
        settle(sb, pb, step(kNext{}, kDyn{}, s, (s + 1) & 1, sb, sa, pa, pb));
        ++s;
      }
    } else {
      const int ba = (s + 1) & 1;
      for (; s + 1 < ws1; s += 2) {
        step(kNext{}, kDyn{}, s, ba, sa, sb, pb, pa);
        step(kNext{}, kDyn{}, s + 1, ba ^ 1, sb, sa, pa, pb);
      }
      last_in_pa = s < ws1;
      if (s < ws1) {
        step(kNext{}, kDyn{}, s, (s + 1) & 1, sa, sb, pb, pa);
        ++s;
      }
    }
  }
  // the P.V of the wave's last tile (its V, in buffer (ws1 - 1) mod NB, is
  // overwritten only by the loads of step ws1 + 1), then its rows leave while
  // the other waves go on
  // (now: after the loop's last step, the rows are stored at once; before
  // it they are staged and stored after it)
  bool store_owed = false;
  auto drain = [&](bool now) {
    if (ws1 > ws0) {
      const T* vb = vbuf0 + ring(ws1 - 1) * TILE;
      if (last_in_pa) pv_only(vb, pa);
      else pv_only(vb, pb);
    }
    if constexpr (D <= 64) {
      epi_stage(std::true_type{});
      if (now) epi_store();
      else store_owed = true;
    } else if (now) {
      epi_stage(std::true_type{});
      epi_store();
    } else {
      store_owed = true;  // normalised, staged and stored after the last barrier
    }
  };
  // the first step after the wave's own (step ws1, or step 0 for a wave
  // without keys) brings its last V; it drains there, then only loads (kept
  // out of the loop so that none of the store's addressing is hoisted into it)
  if (s < n_steps) {
    light_step(s);
    ++s;
    drain(false);
    for (; s < n_steps; ++s) light_step(s);
  }
  // the steps' end: every wave's last loads have landed (and the final
  // barrier keeps the LDS alive for the waves still draining)
  wait_vm(WaitAll{});
  __builtin_amdgcn_s_barrier();
  if (ws1 == n_steps && ws1 > ws0) drain(true);
  if (store_owed) {
    if constexpr (D > 64) epi_stage(std::true_type{});
    epi_store();
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

  const Unit w = decode_unit<VARLEN, CAUSAL>(p);
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
  // band of row i: keys [i + shift - window, i + shift] (upper bound only
  // when causal) within [0, kv_len); the tiles [j0, j1) cover the workgroup's
  const int shift = p.bottom_right ? w.kv_len - w.q_len : 0;
  const int window = p.window_left < 0 ? (1 << 29) : p.window_left;
  const int kv_end = CAUSAL ? min(w.kv_len, max(blk_last_q + shift + 1, 0)) : w.kv_len;
  const int kv_begin = min(kv_end, max(w.qt * BM + shift - window, 0));
  const int j0 = kv_begin / BN, j1 = kv_end > kv_begin ? (kv_end + BN - 1) / BN : j0;
  const int wave_last = min(row0 + 31, w.q_len - 1);
  const int wave_kv_end = CAUSAL ? min(w.kv_len, max(wave_last + shift + 1, 0)) : w.kv_len;
  const int wave_kv_begin = max(row0 + shift - window, 0);

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

  if (j1 > j0) {
    load_tile(j0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = j0; j < j1; ++j) {
    const int buf = (j - j0) & 1;
    if (j + 1 < j1) load_tile(j + 1);
    const int kbase = j * BN;
    if (wave_active && kbase < wave_kv_end && kbase + BN > wave_kv_begin) {
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
      const bool cut_causal = CAUSAL && kbase + BN - 1 > row0 + shift;
      const bool cut_left = kbase < wave_last + shift - window;
      const bool cut_end = kbase + BN > w.kv_len;
      if (cut_causal || cut_left || cut_end)
        mask_tile<CAUSAL>(s, kbase, qi, w.kv_len, hf, shift, window, cut_causal, cut_left,
                          cut_end);
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
    if (j + 1 < j1) store_tile(buf ^ 1);
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
  // fp16/bf16 kernels run 8-wave workgroups over two query tiles; the fp32
  // kernel runs 4-wave workgroups.
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

int compute_units() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDev && (n = cache[dev].load(std::memory_order_relaxed)) > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < kMaxDev && n > 0) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_fwd(const FwdParams& p, Dt dt, int d, bool causal, bool varlen,
                      hipStream_t stream) {
  const void* fn = d == 64 ? pick_kernel<64>(dt, causal, varlen)
                           : pick_kernel<128>(dt, causal, varlen);
  if (!fn) return hipErrorInvalidValue;
  // fp16/bf16: units are pairs of query tiles, two 4-wave workgroups each
  // (d = 64, causal) or one 8-wave workgroup (non-causal d = 128)
  const bool paired = dt != Dt::F32;
  const bool split = paired && (d <= 64 || causal);
  const long long units =
      varlen ? packed_units_per_head(p.total_q, p.b, paired ? 2 * kFwdBlockM : kFwdBlockM) * p.h
             : (long long)(paired ? (p.n_qtiles + 1) / 2 : p.n_qtiles) * p.b * p.h;
  if (units <= 0) return hipSuccess;
  const long long grid = split ? 2 * units : units;
  if (grid > INT_MAX) return hipErrorInvalidValue;
  FwdParams arg = p;
  if (split) {
    const int cus = compute_units();
    if (cus <= 0) return hipErrorInvalidDevice;
    arg.split_round = cus;
  }
  void* args[] = {&arg};
  return hipLaunchKernel(fn, dim3((unsigned)grid),
                         dim3(paired ? fwd16_threads(d, causal) : kFwdThreads), args, 0, stream);
}

}  // namespace sdpa07
