// Device helpers shared by the forward and backward kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace sdpa07 {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLn2 = 0.693147180559945309f;
// Buffer resource word 3 for raw (untyped) loads on gfx9-family parts.
constexpr int kBufferFlags = 0x00020000;
// Cache-policy operand of a buffer store: sc0 | sc1 (system scope).
constexpr int kCacheSystemScope = 1 | 16;
typedef int i32x4 __attribute__((ext_vector_type(4)));

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

// One 16-byte-per-lane buffer load into LDS: lane l's 16 bytes land at LDS
// byte address lds_addr + 16 l. Written as inline assembly so that the
// compiler does not treat later LDS reads as dependent on it (it would wait
// for every such load before each transposing read); the kernels place the
// vmcnt waits themselves. M0, which the instruction takes its LDS address
// from, is saved and restored around it. The descriptor, the scalar offset
// and the LDS address are wave-uniform by the callers' construction; they
// pass through readfirstlane so that the scalar operands stay scalar
// whatever the compiler's uniformity analysis concludes (a no-op on values
// already in scalar registers).
__device__ __forceinline__ void lds_dma16(i32x4 rsrc, int voff, int soff, unsigned lds_addr) {
  const i32x4 rs = {__builtin_amdgcn_readfirstlane(rsrc[0]), __builtin_amdgcn_readfirstlane(rsrc[1]),
                    __builtin_amdgcn_readfirstlane(rsrc[2]), __builtin_amdgcn_readfirstlane(rsrc[3])};
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rs), "s"(__builtin_amdgcn_readfirstlane(soff)),
        "s"(__builtin_amdgcn_readfirstlane(lds_addr))
      : "memory");
}

// A wave-uniform pointer as a fresh scalar value: read from the first lane
// and passed through an empty asm, so that address arithmetic on it is
// done where it is used and not shared with (or hoisted to) earlier code.
template <typename P>
__device__ __forceinline__ P* fresh_uniform(P* ptr) {
  const unsigned long long a = (unsigned long long)ptr;
  unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  asm volatile("" : "+s"(lo), "+s"(hi));
  return (P*)(((unsigned long long)hi << 32) | lo);
}

// Value of x held by the lane 32 positions away (the other half-wave).
__device__ __forceinline__ float other_half(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  // Lanes < 32 receive the upper half in sw[1]; lanes >= 32 the lower in sw[0].
  const unsigned o = (threadIdx.x & 32) ? sw[0] : sw[1];
  return __builtin_bit_cast(float, o);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Pins the computation of x before this point of the instruction stream (an
// empty volatile asm that reads x: volatile asms keep their order, so x's
// producers cannot sink past it). Used to keep softmax work interleaved with
// the MFMAs it is meant to overlap.
template <typename X>
__device__ __forceinline__ void pin(const X& x) {
  asm volatile("" ::"v"(x));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

typedef float f32x2 __attribute__((ext_vector_type(2)));

template <typename T>
struct Pack2;
template <>
struct Pack2<__bf16> {
  using type = bf16x2;
};
template <>
struct Pack2<_Float16> {
  using type = f16x2;
};

// acc + h.x + h.y for a packed pair of 16-bit values (one v_dot2 with ones).
template <typename T>
__device__ __forceinline__ float dot2_ones(typename Pack2<T>::type h, float acc);
template <>
__device__ __forceinline__ float dot2_ones<__bf16>(bf16x2 h, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(h, one, acc, false);
}
template <>
__device__ __forceinline__ float dot2_ones<_Float16>(f16x2 h, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(h, one, acc, false);
}

// ---- live work units of a packed (THD) batch, heaviest first ---------------
//
// The grid of a packed launch is sized from totals the host knows (for
// example total_q / 256 + num_seqs pairs of query tiles per head), never
// from the lengths, which only the device holds. Each workgroup then finds
// its own unit: sequence s holds n_s units, and unit j of it costs a_s - j
// (taper: the causal tiles, whose key ranges shrink with j; a_s >= n_s) or
// a_s (flat). Units are taken in decreasing order of cost (ties by sequence,
// then j), so the longest start first and the last to start are short. The
// rank u of a unit in that order is inverted by a binary search on the cost:
// C(k) = number of units costing at least k, a sum over sequences taken 64
// at a time with one wave reduction; then the sequence holding the
// (u - C(k* + 1))-th unit of cost k* by a prefix sum. Ranks past the last
// unit give seq = -1. Every lane of the calling wave takes part and receives
// the same result.
struct PackedUnit {
  int seq;
  int j;
};

// (the totals are returned through readfirstlane, so that the compiler
// keeps them, and the control flow that depends on them, scalar)
__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o);
  return __builtin_amdgcn_readfirstlane(x);
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = max(x, __shfl_xor(x, o));
  return __builtin_amdgcn_readfirstlane(x);
}
__device__ __forceinline__ int wave_incl_scan_i(int x) {
  const int lane = threadIdx.x % 64;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// units_of(s) returns int2{n_s, a_s} for sequence s < nseq.
template <typename F>
__device__ PackedUnit packed_unit(int u, int nseq, bool taper, F&& units_of) {
  const int lane = threadIdx.x % 64;
  auto cnt = [&](int n, int a, int k) -> int {
    return taper ? min(max(a - k + 1, 0), n) : (a >= k ? n : 0);
  };
  // the first 64 sequences are read once; later ones on every pass
  int n0 = 0, a0 = 0;
  if (lane < nseq) {
    const int2 na = units_of(lane);
    n0 = na.x;
    a0 = na.y;
  }
  auto count_ge = [&](int k) -> int {
    int c = cnt(n0, a0, k);
    for (int s0 = 64; s0 < nseq; s0 += 64) {
      if (s0 + lane < nseq) {
        const int2 na = units_of(s0 + lane);
        c += cnt(na.x, na.y, k);
      }
    }
    return wave_sum_i(c);
  };
  int amax = n0 > 0 ? a0 : 0;
  for (int s0 = 64; s0 < nseq; s0 += 64) {
    if (s0 + lane < nseq) {
      const int2 na = units_of(s0 + lane);
      if (na.x > 0) amax = max(amax, na.y);
    }
  }
  amax = wave_max_i(amax);
  if (amax <= 0 || u >= count_ge(1)) return {-1, 0};
  int lo = 1, hi = amax;  // C(lo) > u >= C(hi + 1)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (count_ge(mid) > u) lo = mid;
    else hi = mid - 1;
  }
  int r = u - count_ge(lo + 1);  // rank among the units of cost exactly lo
  for (int s0 = 0; s0 < nseq; s0 += 64) {
    int n = n0, a = a0;
    if (s0 > 0) {
      n = a = 0;
      if (s0 + lane < nseq) {
        const int2 na = units_of(s0 + lane);
        n = na.x;
        a = na.y;
      }
    }
    const int e = cnt(n, a, lo) - cnt(n, a, lo + 1);
    const int incl = wave_incl_scan_i(e);
    const int tot = __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
    if (r < tot) {
      const unsigned long long m = __ballot(incl > r);
      const int first = __builtin_amdgcn_readfirstlane(__ffsll((long long)m) - 1);
      const int excl = __builtin_amdgcn_readfirstlane(__shfl(incl - e, first));
      const int af = __builtin_amdgcn_readfirstlane(__shfl(a, first));
      return {s0 + first, taper ? af - lo : r - excl};
    }
    r -= tot;
  }
  return {-1, 0};
}

// Clamped length of packed sequence s: cu[s + 1] - cu[s] within [0, total].
__device__ __forceinline__ int packed_len(const int32_t* cu, int s, int total) {
  const int a = min(max(cu[s], 0), total);
  const int b = min(max(cu[s + 1], 0), total);
  return max(b - a, 0);
}

// Stores the 32 x D tile that a wave holds in the C layout of a transposed
// product (lane: row lane % 32; register 4 rq + e of block db: column
// 32 db + 8 rq + 4 (lane / 32) + e), scaled by f, as whole rows: the pieces
// go into the wave's LDS area stg ([32][D], 16-byte chunks XOR-permuted by
// the row), each lane reads back whole chunks, and each store instruction
// writes 64 / (D / 8) complete rows with the system-scope cache policy
// (written through as stored). Rows from n_rows on are dropped by the
// descriptor's byte bound. base: row 0; row_stride in elements, below 2^24
// (the caller's check). The LDS area must be free for the wave's use.
template <typename T, int D>
__device__ __forceinline__ void store_rows_via_lds(T* stg, const f32x16 (&x)[D / 32], float f,
                                                   T* base, int64_t row_stride, int n_rows,
                                                   int lane) {
  typedef T t4 __attribute__((ext_vector_type(4)));
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int RPS = 64 / CPR;  // rows per store instruction
  const int cl = lane % 32, hl = lane / 32;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      t4 ov;
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = (T)(x[db][4 * rq + e] * f);
      *(t4*)&stg[cl * D + ((4 * db + rq) ^ (cl % CPR)) * 8 + 4 * hl] = ov;
    }
  // the wave reads back what its other lanes wrote (LDS operations of one
  // wave complete in order; the fences keep the compiler's order and wait)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int sr = lane / CPR, sc = lane % CPR;
  i32x4 v[32 / RPS];
#pragma unroll
  for (int xi = 0; xi < 32 / RPS; ++xi) {
    const int r = xi * RPS + sr;
    v[xi] = *(const i32x4*)&stg[r * D + (sc ^ (r % CPR)) * 8];
  }
  const int rows = min(max(n_rows, 0), 32);
  const int bytes = rows == 0 ? 0 : ((rows - 1) * (int)row_stride + D) * (int)sizeof(T);
  const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, kBufferFlags);
  const int voff = (sr * (int)row_stride + sc * 8) * (int)sizeof(T);
#pragma unroll
  for (int xi = 0; xi < 32 / RPS; ++xi)
    __builtin_amdgcn_raw_buffer_store_b128(v[xi], rs, voff,
                                           xi * RPS * (int)row_stride * (int)sizeof(T),
                                           kCacheSystemScope);
}

}  // namespace
}  // namespace sdpa07
