// fmm_device.h -- device helpers for the gfx950 kernels: wave64 primitives,
// Morton bit spreading, compile-time multi-index tables.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>
#include <utility>

namespace mbg {

constexpr int WAVE = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }
__device__ __forceinline__ uint64_t lanemask_lt() {
  return (1ull << __lane_id()) - 1ull;
}

// Value of lane 0 in a scalar register (for values known to be wave-uniform).
__device__ __forceinline__ int32_t uniform(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform(int64_t v) {
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Issue priority of a wave among those on its SIMD.  The short, latency-bound
// kernels that build the lists and tasks can run beside the ALU-bound sibling
// M2L on the other stream; raising their waves' priority lets their few
// instructions through ahead of the M2L's long arithmetic stream.
__device__ __forceinline__ void bookkeeping_priority() { __builtin_amdgcn_s_setprio(3); }

// ---- cross-lane moves inside rows of 16 lanes (DPP), no LDS round trip ----
// DPP controls: quad_perm, row_shr:n, row_mirror, row_half_mirror.  A lane
// whose source lies outside its row receives 0.
constexpr int DPP_QUAD_XOR1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int dpp_row_shr(int n) { return 0x110 + n; }

template <int CTRL>
__device__ __forceinline__ int32_t dpp_move(int32_t v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, true);
}
template <int CTRL>
__device__ __forceinline__ int64_t dpp_move(int64_t v) {
  const uint32_t lo = (uint32_t)dpp_move<CTRL>((int32_t)(uint32_t)(uint64_t)v);
  const uint32_t hi = (uint32_t)dpp_move<CTRL>((int32_t)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_move(uint64_t v) {
  return (uint64_t)dpp_move<CTRL>((int64_t)v);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v) {
  return (uint32_t)dpp_move<CTRL>((int32_t)v);
}
template <int CTRL>
__device__ __forceinline__ double dpp_move(double v) {
  return __longlong_as_double((long long)dpp_move<CTRL>((int64_t)__double_as_longlong(v)));
}
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(dpp_move<CTRL>((int32_t)__float_as_int(v)));
}
__device__ __forceinline__ int32_t read_lane(int32_t v, int l) {
  return __builtin_amdgcn_readlane(v, l);
}
__device__ __forceinline__ uint32_t read_lane(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int32_t)v, l);
}
__device__ __forceinline__ int64_t read_lane(int64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int32_t)(uint32_t)(uint64_t)v, l);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_readlane((int32_t)(uint32_t)((uint64_t)v >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint64_t read_lane(uint64_t v, int l) {
  return (uint64_t)read_lane((int64_t)v, l);
}

// Wave-wide sum of an integer type (all 64 lanes active): butterflies inside
// each row, then the four row sums; every lane gets the same value.
template <typename I>
__device__ __forceinline__ I wave_sum(I v) {
  static_assert(std::is_integral<I>::value, "integer sums only");
  v += dpp_move<DPP_QUAD_XOR1>(v);
  v += dpp_move<DPP_QUAD_XOR2>(v);
  v += dpp_move<DPP_ROW_HALF_MIRROR>(v);
  v += dpp_move<DPP_ROW_MIRROR>(v);
  return (read_lane(v, 0) + read_lane(v, 16)) + (read_lane(v, 32) + read_lane(v, 48));
}

// Inclusive prefix sum over the wave (integer types, all 64 lanes active):
// shifts by 1, 2, 4, 8 inside each row of 16, then each row adds the totals
// of the rows before it.
template <typename I>
__device__ __forceinline__ I wave_incl_scan(I v) {
  static_assert(std::is_integral<I>::value, "integer scans only");
  v += dpp_move<dpp_row_shr(1)>(v);
  v += dpp_move<dpp_row_shr(2)>(v);
  v += dpp_move<dpp_row_shr(4)>(v);
  v += dpp_move<dpp_row_shr(8)>(v);
  const I r0 = read_lane(v, 15), r1 = read_lane(v, 31), r2 = read_lane(v, 47);
  const int row = __lane_id() >> 4;
  I add = 0;
  if (row >= 1) add += r0;
  if (row >= 2) add += r1;
  if (row >= 3) add += r2;
  return v + add;
}

// Launch-order octave of a work estimate w: 63 - floor(log2 w), 63 for w = 0
// (so ascending octaves are descending work).
__device__ __forceinline__ int work_octave(uint64_t w) {
  return 63 - (w ? 63 - __clzll(w) : 0);
}

// Block-wide placement into octave buckets (blockDim.x threads, all calling):
// returns this thread's slot for octave o (o < 0: none).  oct[] holds the
// bucket sizes of the whole launch, cur[] global cursors (zero at the start);
// a block takes one contiguous range per bucket, so items of one block stay
// together, in an order that depends on timing only inside the block.
template <int NB>
__device__ __forceinline__ int64_t octave_slot(int o, const int32_t* oct, int32_t* cur) {
  __shared__ int cnt[NB];
  __shared__ int tot[NB];  // the buckets' totals, staged once per block
  __shared__ int64_t base[NB];
  for (int b = threadIdx.x; b < NB; b += blockDim.x) {
    cnt[b] = 0;
    tot[b] = oct[b];
  }
  __syncthreads();
  const int r = o >= 0 ? atomicAdd(&cnt[o], 1) : 0;
  __syncthreads();
  for (int b = threadIdx.x; b < NB; b += blockDim.x) {
    int64_t start = 0;
    for (int q = 0; q < b; q++) start += tot[q];
    base[b] = cnt[b] ? start + atomicAdd(&cur[b], cnt[b]) : 0;
  }
  __syncthreads();
  return o >= 0 ? base[o] + r : -1;
}

// Spread the low 21 bits of v to every third bit (bit b -> bit 3b).
__device__ __forceinline__ uint64_t spread3(uint32_t v) {
  uint64_t x = v & 0x1fffffull;
  x = (x | (x << 32)) & 0x001f00000000ffffull;
  x = (x | (x << 16)) & 0x001f0000ff0000ffull;
  x = (x | (x << 8)) & 0x100f00f00f00f00full;
  x = (x | (x << 4)) & 0x10c30c30c30c30c3ull;
  x = (x | (x << 2)) & 0x1249249249249249ull;
  return x;
}
// Inverse of spread3: gather every third bit (bit 3b -> bit b).
__host__ __device__ __forceinline__ uint32_t compact3(uint64_t x) {
  x &= 0x1249249249249249ull;
  x = (x ^ (x >> 2)) & 0x10c30c30c30c30c3ull;
  x = (x ^ (x >> 4)) & 0x100f00f00f00f00full;
  x = (x ^ (x >> 8)) & 0x001f0000ff0000ffull;
  x = (x ^ (x >> 16)) & 0x001f00000000ffffull;
  x = (x ^ (x >> 32)) & 0x1fffffull;
  return (uint32_t)x;
}

// Deepest level at which two keys share a cell (21 if equal).
__device__ __forceinline__ int shared_level(uint64_t a, uint64_t b) {
  uint64_t x = a ^ b;
  if (x == 0) return 21;
  return (__clzll(x) - 1) / 3;  // bit 63 of a key is always 0
}

// ---- multi-indices (a,b,c), |.| <= p, graded: degree, then a desc, b desc ----
__host__ __device__ constexpr int mi_index(int a, int b, int c) {
  int d = a + b + c;
  return d * (d + 1) * (d + 2) / 6 + (b + c) * (b + c + 1) / 2 + c;
}

template <int P>
struct MI {
  static constexpr int K = (P + 1) * (P + 2) * (P + 3) / 6;
  int a[K], b[K], c[K], d[K];
  constexpr MI() : a(), b(), c(), d() {
    int k = 0;
    for (int dd = 0; dd <= P; dd++)
      for (int aa = dd; aa >= 0; aa--)
        for (int bb = dd - aa; bb >= 0; bb--) {
          a[k] = aa;
          b[k] = bb;
          c[k] = dd - aa - bb;
          d[k] = dd;
          k++;
        }
  }
};

// Compile-time loop: f(std::integral_constant<int, i>) for i = B .. E-1, in order.
template <int B, typename F, int... I>
__host__ __device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, B + I>{}), ...);
}
template <int B, int E, typename F>
__host__ __device__ __forceinline__ void static_for(F&& f) {
  if constexpr (E - B <= 512) {
    static_for_impl<B>(f, std::make_integer_sequence<int, E - B>{});
  } else {
    constexpr int M = B + (E - B) / 2;
    static_for<B, M>(f);
    static_for<M, E>(f);
  }
}

__host__ __device__ constexpr int binom_c(int n, int k) {
  int r = 1;
  for (int i = 1; i <= k; i++) r = r * (n - k + i) / i;
  return r;
}

// Tables for order P, usable as constant expressions in device code:
//   coefficient k <-> (a, b, c);
//   contraction triples (n, m, n+m) with |n| + |m| <= P;
//   the derivative recurrence over levels j = P .. 0, flattened: entry e of
//   level j (multi-index k, |k| <= P - j) is built from two entries of level j+1.
template <int P>
struct Tabs {
  static constexpr int K = (P + 1) * (P + 2) * (P + 3) / 6;
  static constexpr int NT = binom_c(P + 6, 6);
  static constexpr int NR = binom_c(P + 4, 4);
  int a[K], b[K], c[K], d[K];
  int tn[NT], tm[NT], tk[NT];
  int roff[P + 2];           // flat offset of level j
  int rlev[NR], rk[NR];      // level and multi-index of every flat entry
  int raxis[NR];             // -1: level head g_j; else axis 0/1/2
  int rs1[NR], rs2[NR];      // flat sources (rs2 = -1 when absent)
  int rc2[NR];               // integer factor of the second source
  constexpr Tabs()
      : a(), b(), c(), d(), tn(), tm(), tk(), roff(), rlev(), rk(), raxis(), rs1(), rs2(), rc2() {
    int k = 0;
    for (int dd = 0; dd <= P; dd++)
      for (int aa = dd; aa >= 0; aa--)
        for (int bb = dd - aa; bb >= 0; bb--) {
          a[k] = aa;
          b[k] = bb;
          c[k] = dd - aa - bb;
          d[k] = dd;
          k++;
        }
    int t = 0;
    for (int n = 0; n < K; n++)
      for (int m = 0; m < K; m++)
        if (d[n] + d[m] <= P) {
          tn[t] = n;
          tm[t] = m;
          tk[t] = mi_index(a[n] + a[m], b[n] + b[m], c[n] + c[m]);
          t++;
        }
    // level j has C(P-j+3,3) entries; levels stored from j = P down to 0
    int off = 0;
    for (int j = P; j >= 0; j--) {
      roff[j] = off;
      off += binom_c(P - j + 3, 3);
    }
    roff[P + 1] = 0;
    for (int j = P; j >= 0; j--) {
      int n_j = binom_c(P - j + 3, 3);
      for (int q = 0; q < n_j; q++) {
        int e = roff[j] + q;
        rlev[e] = j;
        rk[e] = q;
        if (q == 0) {
          raxis[e] = -1;
          rs1[e] = rs2[e] = -1;
          rc2[e] = 0;
          continue;
        }
        int ka = a[q], kb = b[q], kc = c[q];
        int ax = ka > 0 ? 0 : (kb > 0 ? 1 : 2);
        int ia = ka, ib = kb, ic = kc;  // k - e_ax
        if (ax == 0) ia--;
        if (ax == 1) ib--;
        if (ax == 2) ic--;
        raxis[e] = ax;
        rs1[e] = roff[j + 1] + mi_index(ia, ib, ic);
        int prev = ax == 0 ? ia : (ax == 1 ? ib : ic);  // (k - e_ax)_ax
        if (prev > 0) {
          rs2[e] = roff[j + 1] + mi_index(ia - (ax == 0), ib - (ax == 1), ic - (ax == 2));
          rc2[e] = prev;
        } else {
          rs2[e] = -1;
          rc2[e] = 0;
        }
      }
    }
  }
};

template <int P>
inline constexpr Tabs<P> tabs{};

// Tables for the traceless form of the translation.  The derivatives of 1/r
// are harmonic: D_(k+2x) + D_(k+2y) + D_(k+2z) = 0.  So a moment component
// with m_z >= 2 can be folded onto m - 2z + 2x and m - 2z + 2y (with sign -1)
// without changing any sum_m Mt_m D_(n+m) -- the degree |m| is kept, so the
// truncation |n| + |m| <= P is kept too -- and a local coefficient with
// n_z >= 2 follows from two with one less z:  L_n = -L_(n-2z+2x) - L_(n-2z+2y).
// The translation then runs over n, m with n_z, m_z <= 1 only: (P+1)^2
// components each instead of C(P+3,3).
//   rfull[r]          full index of reduced component r (graded order kept)
//   tn, tm, tk        contraction terms: reduced n, reduced m, full n+m
//   fold (dst, src)   moment folding, in an order that finishes every source
//   rec (dst, s1, s2) local reconstruction, in increasing n_z
template <int P>
struct HTabs {
  static constexpr int K = (P + 1) * (P + 2) * (P + 3) / 6;
  static constexpr int KR = (P + 1) * (P + 1);
  static constexpr int NF = 2 * (K - KR);
  static constexpr int NRC = K - KR;
  static constexpr int count_terms() {
    int t = 0;
    for (int dn = 0; dn <= P; dn++)
      for (int dm = 0; dm + dn <= P; dm++) t += (2 * dn + 1) * (2 * dm + 1);
    return t;
  }
  static constexpr int NT = count_terms();
  int rfull[KR];
  int tn[NT], tm[NT], tk[NT];
  int ko[K + 1];        // the terms grouped by derivative index: terms of k are
  int kn[NT], km[NT];   //   (kn, km)[ko[k] .. ko[k+1])
  int fd[NF], fs[NF];
  int rd[NRC], r1[NRC], r2[NRC];
  constexpr HTabs()
      : rfull(), tn(), tm(), tk(), ko(), kn(), km(), fd(), fs(), rd(), r1(), r2() {
    int a[K] = {}, b[K] = {}, c[K] = {}, d[K] = {};
    int k = 0;
    for (int dd = 0; dd <= P; dd++)
      for (int aa = dd; aa >= 0; aa--)
        for (int bb = dd - aa; bb >= 0; bb--) {
          a[k] = aa;
          b[k] = bb;
          c[k] = dd - aa - bb;
          d[k] = dd;
          k++;
        }
    int red[K] = {};
    int r = 0;
    for (int q = 0; q < K; q++) {
      red[q] = -1;
      if (c[q] <= 1) {
        rfull[r] = q;
        red[q] = r;
        r++;
      }
    }
    int t = 0;
    for (int n = 0; n < K; n++)
      for (int m = 0; m < K; m++)
        if (c[n] <= 1 && c[m] <= 1 && d[n] + d[m] <= P) {
          tn[t] = red[n];
          tm[t] = red[m];
          tk[t] = mi_index(a[n] + a[m], b[n] + b[m], c[n] + c[m]);
          t++;
        }
    int o = 0;
    for (int kk = 0; kk < K; kk++) {
      ko[kk] = o;
      for (int q = 0; q < t; q++)
        if (tk[q] == kk) {
          kn[o] = tn[q];
          km[o] = tm[q];
          o++;
        }
    }
    ko[K] = o;
    // folding: sources with the largest z first (their targets have z - 2)
    int f = 0;
    for (int cz = P; cz >= 2; cz--)
      for (int q = 0; q < K; q++)
        if (c[q] == cz) {
          fd[f] = mi_index(a[q] + 2, b[q], c[q] - 2);
          fs[f] = q;
          f++;
          fd[f] = mi_index(a[q], b[q] + 2, c[q] - 2);
          fs[f] = q;
          f++;
        }
    // reconstruction: increasing z, so both sources are known
    int e = 0;
    for (int cz = 2; cz <= P; cz++)
      for (int q = 0; q < K; q++)
        if (c[q] == cz) {
          rd[e] = q;
          r1[e] = mi_index(a[q] + 2, b[q], c[q] - 2);
          r2[e] = mi_index(a[q], b[q] + 2, c[q] - 2);
          e++;
        }
  }
};

template <int P>
inline constexpr HTabs<P> htabs{};

template <typename T>
struct alignas(4 * sizeof(T)) P4 {
  T x, y, z, m;
};
// A particle with its VJP sensitivities: position and mass, then pb = dS/dphi
// and ab = dS/da.
template <typename T>
struct alignas(8 * sizeof(T)) P8 {
  P4<T> p;  // x, y, z, m
  P4<T> c;  // pb, abx, aby, abz
};

}  // namespace mbg
