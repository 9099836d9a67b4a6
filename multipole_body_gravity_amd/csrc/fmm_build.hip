// fmm_build.hip -- build-stage kernels: bounding box, Morton keys, LSD radix
// sort, gather into sorted order, device-wide scans and the octree.
//
// The jz-fmm project page ("Why this works well on GPUs") keeps sorting and tree
// construction on the GPU with neighbouring particles and sibling nodes next to
// each other in memory; the layout rules (root cube, 21-bit keys, leaf rule,
// breadth-first numbering) are documented in include/fmm.h.
#include <atomic>
#include "fmm_device.h"
#include "fmm_internal.h"

namespace mbg {

// ===================================================================
// device-wide exclusive scan (reduce -> scan block sums -> apply)
// ===================================================================
constexpr int SCAN_THREADS = 256;
constexpr int SCAN_ITEMS = 8;
constexpr int SCAN_TILE = SCAN_THREADS * SCAN_ITEMS;
constexpr int64_t SCAN_DIRECT_BLOCKS = 2048;  // up to here blocks sum their offsets themselves

template <typename I>
__device__ I block_excl_scan(I v, I* total) {
  __shared__ I wsum[SCAN_THREADS / WAVE];
  const int w = threadIdx.x / WAVE, l = threadIdx.x % WAVE;
  I inc = wave_incl_scan(v);
  if (l == WAVE - 1) wsum[w] = inc;
  __syncthreads();
  I off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < SCAN_THREADS / WAVE; i++) {
    if (i < w) off += wsum[i];
    tot += wsum[i];
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

template <typename I>
__global__ void __launch_bounds__(SCAN_THREADS) k_scan_reduce(const I* in, int64_t n, I* sums) {
  bookkeeping_priority();
  int64_t base = (int64_t)blockIdx.x * SCAN_TILE + (int64_t)threadIdx.x * SCAN_ITEMS;
  I s = 0;
#pragma unroll
  for (int i = 0; i < SCAN_ITEMS; i++)
    if (base + i < n) s += in[base + i];
  I tot;
  block_excl_scan(s, &tot);
  if (threadIdx.x == 0) sums[blockIdx.x] = tot;
}

template <typename I>
__global__ void __launch_bounds__(SCAN_THREADS) k_scan_top(I* sums, int64_t nb, I* total) {
  bookkeeping_priority();
  __shared__ I carry_s;
  if (threadIdx.x == 0) carry_s = 0;
  __syncthreads();
  for (int64_t base = 0; base < nb; base += SCAN_THREADS) {
    int64_t i = base + threadIdx.x;
    I v = i < nb ? sums[i] : 0;
    I tot;
    I ex = block_excl_scan(v, &tot);
    I c = carry_s;
    if (i < nb) sums[i] = c + ex;
    __syncthreads();
    if (threadIdx.x == 0) carry_s = c + tot;
    __syncthreads();
  }
  if (threadIdx.x == 0 && total) *total = carry_s;
}

template <typename I>
__global__ void __launch_bounds__(SCAN_THREADS) k_scan_apply(const I* in, I* out, int64_t n,
                                                             const I* sums) {
  bookkeeping_priority();
  int64_t base = (int64_t)blockIdx.x * SCAN_TILE + (int64_t)threadIdx.x * SCAN_ITEMS;
  I v[SCAN_ITEMS];
  I s = 0;
#pragma unroll
  for (int i = 0; i < SCAN_ITEMS; i++) {
    v[i] = (base + i < n) ? in[base + i] : 0;
    s += v[i];
  }
  I tot;
  I ex = block_excl_scan(s, &tot) + sums[blockIdx.x];
#pragma unroll
  for (int i = 0; i < SCAN_ITEMS; i++) {
    if (base + i < n) out[base + i] = ex;
    ex += v[i];
  }
}

// Apply with the block offsets summed in place: block b adds sums[0 .. b-1]
// itself (a few thousand block sums at most), so no separate pass scans them;
// sums == null means a single block.  The last block writes the total.
template <typename I>
__global__ void __launch_bounds__(SCAN_THREADS) k_scan_apply_direct(const I* in, I* out, int64_t n,
                                                                    const I* sums, I* total) {
  bookkeeping_priority();
  I part = 0;
  if (sums)
    for (int64_t i = threadIdx.x; i < (int64_t)blockIdx.x; i += SCAN_THREADS) part += sums[i];
  I boff;
  block_excl_scan(part, &boff);
  const int64_t base = (int64_t)blockIdx.x * SCAN_TILE + (int64_t)threadIdx.x * SCAN_ITEMS;
  I v[SCAN_ITEMS];
  I s = 0;
#pragma unroll
  for (int i = 0; i < SCAN_ITEMS; i++) {
    v[i] = (base + i < n) ? in[base + i] : 0;
    s += v[i];
  }
  I tot;
  I ex = block_excl_scan(s, &tot) + boff;
#pragma unroll
  for (int i = 0; i < SCAN_ITEMS; i++) {
    if (base + i < n) out[base + i] = ex;
    ex += v[i];
  }
  if (total && blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) *total = boff + tot;
}

size_t scan_tmp_bytes(int64_t n) {
  int64_t nb = (n + SCAN_TILE - 1) / SCAN_TILE;
  return (size_t)(nb + 1) * sizeof(int64_t);
}

template <typename I>
__global__ void k_set_zero(I* p) {
  bookkeeping_priority();
  if (threadIdx.x == 0) *p = 0;
}

template <typename I>
static hipError_t scan_excl(const I* in, I* out, int64_t n, I* total, void* tmp, hipStream_t st) {
  if (n <= 0) {
    if (total) k_set_zero<I><<<1, 64, 0, st>>>(total);
    return hipGetLastError();
  }
  int64_t nb = (n + SCAN_TILE - 1) / SCAN_TILE;
  I* sums = (I*)tmp;
  if (nb == 1) {
    k_scan_apply_direct<I><<<1, SCAN_THREADS, 0, st>>>(in, out, n, nullptr, total);
    return hipGetLastError();
  }
  k_scan_reduce<I><<<(unsigned)nb, SCAN_THREADS, 0, st>>>(in, n, sums);
  if (nb <= SCAN_DIRECT_BLOCKS) {
    k_scan_apply_direct<I><<<(unsigned)nb, SCAN_THREADS, 0, st>>>(in, out, n, sums, total);
  } else {
    k_scan_top<I><<<1, SCAN_THREADS, 0, st>>>(sums, nb, total);
    k_scan_apply<I><<<(unsigned)nb, SCAN_THREADS, 0, st>>>(in, out, n, sums);
  }
  return hipGetLastError();
}

// ---- up to 3 int64 arrays of one length scanned together ----
// Exclusive scans of in[r] into out[r] (in place allowed), total of array r at
// out[r][n] and, when given, also at dst[r] (a control-block field).
template <int R>
struct ScanMulti {
  const int64_t* in[R];
  int64_t* out[R];
  int64_t* dst[R];
};

template <int R>
__global__ void __launch_bounds__(SCAN_THREADS) k_scan_multi_reduce(ScanMulti<R> a, int64_t n,
                                                                    int64_t* sums) {
  bookkeeping_priority();
  const int64_t base = (int64_t)blockIdx.x * SCAN_TILE + (int64_t)threadIdx.x * SCAN_ITEMS;
#pragma unroll
  for (int r = 0; r < R; r++) {
    int64_t s = 0;
#pragma unroll
    for (int i = 0; i < SCAN_ITEMS; i++)
      if (base + i < n) s += a.in[r][base + i];
    int64_t tot;
    block_excl_scan(s, &tot);
    if (threadIdx.x == 0) sums[(int64_t)r * gridDim.x + blockIdx.x] = tot;
  }
}

// each block sums the block totals before it itself (at most a few thousand)
template <int R>
__global__ void __launch_bounds__(SCAN_THREADS) k_scan_multi_apply(ScanMulti<R> a, int64_t n,
                                                                   const int64_t* sums) {
  bookkeeping_priority();
  const int64_t base = (int64_t)blockIdx.x * SCAN_TILE + (int64_t)threadIdx.x * SCAN_ITEMS;
#pragma unroll
  for (int r = 0; r < R; r++) {
    int64_t part = 0;
    if (sums)
      for (int64_t i = threadIdx.x; i < (int64_t)blockIdx.x; i += SCAN_THREADS)
        part += sums[(int64_t)r * gridDim.x + i];
    int64_t boff;
    block_excl_scan(part, &boff);
    int64_t v[SCAN_ITEMS];
    int64_t s = 0;
#pragma unroll
    for (int i = 0; i < SCAN_ITEMS; i++) {
      v[i] = (base + i < n) ? a.in[r][base + i] : 0;
      s += v[i];
    }
    int64_t tot;
    int64_t ex = block_excl_scan(s, &tot) + boff;
#pragma unroll
    for (int i = 0; i < SCAN_ITEMS; i++) {
      if (base + i < n) a.out[r][base + i] = ex;
      ex += v[i];
    }
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) {
      a.out[r][n] = boff + tot;
      if (a.dst[r]) *a.dst[r] = boff + tot;
    }
  }
}

template <int R>
static hipError_t scan_multi(const ScanMulti<R>& a, int64_t n, void* tmp, hipStream_t st) {
  const int64_t nb = std::max<int64_t>((n + SCAN_TILE - 1) / SCAN_TILE, 1);
  if (nb > SCAN_DIRECT_BLOCKS) {  // long arrays: one classic scan per array
    for (int r = 0; r < R; r++) {
      hipError_t e = scan_excl<int64_t>(a.in[r], a.out[r], n, a.out[r] + n, tmp, st);
      if (e != hipSuccess) return e;
      if (a.dst[r]) {
        e = hipMemcpyAsync(a.dst[r], a.out[r] + n, 8, hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess) return e;
      }
    }
    return hipSuccess;
  }
  int64_t* sums = (int64_t*)tmp;
  if (nb > 1) k_scan_multi_reduce<R><<<(unsigned)nb, SCAN_THREADS, 0, st>>>(a, n, sums);
  k_scan_multi_apply<R><<<(unsigned)nb, SCAN_THREADS, 0, st>>>(a, n, nb > 1 ? sums : nullptr);
  return hipGetLastError();
}

hipError_t scan_exclusive_multi_i64(int r, const int64_t* const* in, int64_t* const* out,
                                    int64_t* const* dst, int64_t n, void* tmp, hipStream_t st) {
  switch (r) {
    case 1: {
      ScanMulti<1> a{{in[0]}, {out[0]}, {dst ? dst[0] : nullptr}};
      return scan_multi<1>(a, n, tmp, st);
    }
    case 2: {
      ScanMulti<2> a{{in[0], in[1]}, {out[0], out[1]},
                     {dst ? dst[0] : nullptr, dst ? dst[1] : nullptr}};
      return scan_multi<2>(a, n, tmp, st);
    }
    case 3: {
      ScanMulti<3> a{{in[0], in[1], in[2]}, {out[0], out[1], out[2]},
                     {dst ? dst[0] : nullptr, dst ? dst[1] : nullptr, dst ? dst[2] : nullptr}};
      return scan_multi<3>(a, n, tmp, st);
    }
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t scan_exclusive_i64(const int64_t* in, int64_t* out, int64_t n, int64_t* total,
                              void* tmp, hipStream_t st) {
  return scan_excl<int64_t>(in, out, n, total, tmp, st);
}
hipError_t scan_exclusive_i32(const int32_t* in, int32_t* out, int64_t n, int32_t* total,
                              void* tmp, hipStream_t st) {
  return scan_excl<int32_t>(in, out, n, total, tmp, st);
}

// ===================================================================
// bounding box (exact min / max) and non-finite detection
// ===================================================================
constexpr int BB_THREADS = 256;

// The root cube of a box: anchored at its minimum corner, side the smallest
// power of two >= the largest extent (1 if every extent is 0); scale = 2^21/side.
__device__ RootInfo root_cube(const double (&lo)[3], const double (&hi)[3]) {
  double ext = 0.0;
  for (int a = 0; a < 3; a++) ext = fmax(ext, __dsub_rn(hi[a], lo[a]));
  // smallest power of two >= ext (1 if ext == 0)
  double side = 1.0;
  if (ext > 0.0 && isfinite(ext)) {
    int e;
    double f = frexp(ext, &e);
    side = (f == 0.5) ? ext : ldexp(1.0, e);
  }
  int e2;
  frexp(side, &e2);
  RootInfo r;
  for (int a = 0; a < 3; a++) r.lo[a] = isfinite(lo[a]) ? lo[a] : 0.0;
  r.side = side;
  r.scale = ldexp(1.0, KEY_BITS - (e2 - 1));
  return r;
}

template <typename T>
__global__ void __launch_bounds__(BB_THREADS)
    k_bbox_partial(const T* pos, const T* mass, int64_t n, double* part, Control* ctrl) {
  double lo[3] = {INFINITY, INFINITY, INFINITY}, hi[3] = {-INFINITY, -INFINITY, -INFINITY};
  int bad = 0;
  for (int64_t i = blockIdx.x * (int64_t)BB_THREADS + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * BB_THREADS) {
#pragma unroll
    for (int a = 0; a < 3; a++) {
      double v = (double)pos[3 * i + a];
      bad |= !isfinite(v);
      lo[a] = fmin(lo[a], v);
      hi[a] = fmax(hi[a], v);
    }
    bad |= !isfinite((double)mass[i]);
  }
  __shared__ double s[6][BB_THREADS / WAVE];
  const int w = threadIdx.x / WAVE, l = threadIdx.x % WAVE;
#pragma unroll
  for (int a = 0; a < 3; a++) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      lo[a] = fmin(lo[a], __shfl_xor(lo[a], o, WAVE));
      hi[a] = fmax(hi[a], __shfl_xor(hi[a], o, WAVE));
    }
  }
  if (l == 0) {
    for (int a = 0; a < 3; a++) {
      s[a][w] = lo[a];
      s[3 + a][w] = hi[a];
    }
  }
  if (__ballot(bad) != 0ull && l == 0) atomicOr(&ctrl->nonfinite, 1);
  __syncthreads();
  if (threadIdx.x < 6) {
    double v = s[threadIdx.x][0];
    for (int i = 1; i < BB_THREADS / WAVE; i++)
      v = threadIdx.x < 3 ? fmin(v, s[threadIdx.x][i]) : fmax(v, s[threadIdx.x][i]);
    part[6 * blockIdx.x + threadIdx.x] = v;
  }
}

__global__ void __launch_bounds__(BB_THREADS) k_bbox_final(const double* part, int nblk, RootInfo* root,
                                                          Control* ctrl) {
  __shared__ double s[6][BB_THREADS];
  double l6[6] = {INFINITY, INFINITY, INFINITY, -INFINITY, -INFINITY, -INFINITY};
  for (int b = threadIdx.x; b < nblk; b += BB_THREADS)
    for (int a = 0; a < 3; a++) {
      l6[a] = fmin(l6[a], part[6 * b + a]);
      l6[3 + a] = fmax(l6[3 + a], part[6 * b + 3 + a]);
    }
  for (int a = 0; a < 6; a++) s[a][threadIdx.x] = l6[a];
  __syncthreads();
  for (int h = BB_THREADS / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h)
      for (int a = 0; a < 6; a++)
        s[a][threadIdx.x] = a < 3 ? fmin(s[a][threadIdx.x], s[a][threadIdx.x + h])
                                  : fmax(s[a][threadIdx.x], s[a][threadIdx.x + h]);
    __syncthreads();
  }
  if (threadIdx.x != 0) return;
  const double lo[3] = {s[0][0], s[1][0], s[2][0]}, hi[3] = {s[3][0], s[4][0], s[5][0]};
  const RootInfo r = root_cube(lo, hi);
  *root = r;
  ctrl->root = r;  // the host's copy comes with the control block
}

hipError_t launch_bbox(const void* pos, const void* mass, int64_t n, int dtype, double* part,
                       int nblk, RootInfo* root, Control* ctrl, hipStream_t st) {
  if (dtype == FMM_F64)
    k_bbox_partial<double><<<nblk, BB_THREADS, 0, st>>>((const double*)pos, (const double*)mass, n,
                                                        part, ctrl);
  else
    k_bbox_partial<float><<<nblk, BB_THREADS, 0, st>>>((const float*)pos, (const float*)mass, n,
                                                       part, ctrl);
  k_bbox_final<<<1, BB_THREADS, 0, st>>>(part, nblk, root, ctrl);
  return hipGetLastError();
}

// ===================================================================
// Morton keys: u = floor((x - lo) * 2^21 / side) clamped, bits interleaved
// ===================================================================
// Morton key of particle i (positions in the dtype, widened exactly).
template <typename T>
__device__ __forceinline__ uint64_t morton_key(const T* pos, int64_t i, const RootInfo& root) {
  const double umax = (double)((1u << KEY_BITS) - 1u);
  uint32_t u[3];
#pragma unroll
  for (int a = 0; a < 3; a++) {
    // one rounding in the subtraction; the scale is an exact power of two
    double s = __dsub_rn((double)pos[3 * i + a], root.lo[a]);
    double v = floor(__dmul_rn(s, root.scale));
    v = fmin(fmax(v, 0.0), umax);
    u[a] = (uint32_t)v;
  }
  return (spread3(u[0]) << 2) | (spread3(u[1]) << 1) | spread3(u[2]);
}

template <typename T>
__global__ void k_keys(const T* pos, int64_t n, const RootInfo* root, uint64_t* keys,
                       int32_t* idx) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n) return;
  keys[i] = morton_key(pos, i, *root);
  idx[i] = (int32_t)i;
}

hipError_t launch_keys(const void* pos, int64_t n, int dtype, const RootInfo* root,
                       uint64_t* keys, int32_t* idx, hipStream_t st) {
  unsigned g = (unsigned)((n + 255) / 256);
  if (dtype == FMM_F64)
    k_keys<double><<<g, 256, 0, st>>>((const double*)pos, n, root, keys, idx);
  else
    k_keys<float><<<g, 256, 0, st>>>((const float*)pos, n, root, keys, idx);
  return hipGetLastError();
}

// ===================================================================
// LSD radix sort of (u64 key, i32 index), stable, digits of 8 or 9 bits
// ===================================================================
constexpr int RS_THREADS = 256;
constexpr int RS_MAX_RADIX = 512;
// Keys per thread of a tile: 8 up to 2^23 keys, 16 above.  Each tile is one
// dependent chain (load, rank, reorder, write); with the shorter tiles a sort
// of 10^6 keys has two per compute unit instead of one, whose chains overlap
// (7 % off the 10^6-key sort); at 1.7*10^7 keys and more the longer tiles win
// (half the per-tile histograms to scan).
constexpr int64_t RS_SHORT_TILES_MAX = (int64_t)1 << 23;
static int64_t rs_tile(int64_t n) { return RS_THREADS * (n <= RS_SHORT_TILES_MAX ? 8 : 16); }

size_t radix_hist_ints(int64_t n) {
  const int64_t tile = rs_tile(n);
  int64_t nb = (n + tile - 1) / tile;
  return (size_t)(RS_MAX_RADIX * nb);
}

// digit of key at `shift` (dmask: the pass's digit mask) and the lanes of the
// wave holding the same digit, from RB ballots
template <int RB>
__device__ __forceinline__ uint64_t same_digit(int d, bool valid) {
  uint64_t mask = __ballot(valid);
#pragma unroll
  for (int b = 0; b < RB; b++) {
    const uint64_t bb = __ballot((d >> b) & 1);
    mask &= ((d >> b) & 1) ? bb : ~bb;
  }
  return mask;
}

template <int RB, int RS_ROUNDS>
__global__ void __launch_bounds__(RS_THREADS)
    k_radix_hist(const uint64_t* keys, int64_t n, int shift, uint32_t dmask, int32_t* hist,
                 int nblk, const int64_t* n_dev, const Control* stop) {
  bookkeeping_priority();
  // keys present: n, or min(*n_dev, n), or none after a walk abort (the
  // blocks past the end still write their empty histograms)
  if (n_dev) n = min(*n_dev, n);
  if (stop && walk_aborted(stop)) n = 0;
  constexpr int R = 1 << RB;
  constexpr int RS_TILE = RS_THREADS * RS_ROUNDS;
  __shared__ int h[R];
  for (int d = threadIdx.x; d < R; d += RS_THREADS) h[d] = 0;
  __syncthreads();
  int64_t base = (int64_t)blockIdx.x * RS_TILE;
  int dg[RS_ROUNDS];  // all loads issued before the first use
#pragma unroll
  for (int r = 0; r < RS_ROUNDS; r++) {
    int64_t i = base + r * RS_THREADS + threadIdx.x;
    dg[r] = i < n ? (int)((keys[i] >> shift) & dmask) : -1;
  }
  // one LDS atomic per distinct digit of a wave and round (equal digits found
  // by ballots): few distinct digits do not serialize on one counter
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int r = 0; r < RS_ROUNDS; r++) {
    const int d = dg[r];
    const uint64_t mask = same_digit<RB>(d, d >= 0);
    if (d >= 0 && (mask & lt) == 0) atomicAdd(&h[d], __popcll(mask));
  }
  __syncthreads();
  for (int d = threadIdx.x; d < R; d += RS_THREADS)
    hist[(int64_t)d * nblk + blockIdx.x] = h[d];
}

// Scatter of one tile, stable.  Wave w ranks the w-th quarter of the tile on
// its own, 64 elements per round in input order: ranks among equal digits
// come from wave ballots (lower lanes first) added to the wave's running count
// of the digit.  The per-wave counts are then combined in wave order (earlier
// quarters first) and over digits, the tile is reordered by digit in LDS and
// written out in that order, so each digit's run goes to consecutive addresses.
// LDS of one tile of the scatter: its keys and values reordered by digit,
// the per-wave digit counts (then starts), each digit's start in the tile and
// its global start.
template <int RB, int RS_ROUNDS>
struct RsTile {
  static constexpr int R = 1 << RB;
  static constexpr int TILE = RS_THREADS * RS_ROUNDS;
  static constexpr int NW = RS_THREADS / WAVE;
  uint64_t skey[TILE];
  int32_t sval[TILE];
  int wcnt[NW][R];
  int dstart[R];
  int gbase[R];
  int wsum[NW];
};

// Rank one tile, stable: wave w ranks the w-th quarter of the tile on its own,
// 64 elements per round in input order: ranks among equal digits come from
// wave ballots (lower lanes first) added to the wave's running count of the
// digit.  The per-wave counts are then combined in wave order (earlier
// quarters first) and over digits; the tile is reordered by digit in LDS.
// On return tot[k] is the tile's count of digit DPT tid + k, sh.dstart the
// tile-local start of each digit's run, and the tile sits in sh.skey/sh.sval
// in digit order (a block barrier has passed).
template <int RB, int RS_ROUNDS>
__device__ __forceinline__ void rs_rank_tile(const uint64_t* kin, const int32_t* vin, int64_t n,
                                             int64_t tile, int shift, uint32_t dmask,
                                             RsTile<RB, RS_ROUNDS>& sh,
                                             int (&tot)[(1 << RB) / RS_THREADS]) {
  using S = RsTile<RB, RS_ROUNDS>;
  constexpr int R = S::R, NW = S::NW;
  constexpr int DPT = R / RS_THREADS;  // digits per thread in the digit scan (1 or 2)
  constexpr int WTILE = S::TILE / NW;  // elements per wave
  const int tid = threadIdx.x, w = tid / WAVE, lane = __lane_id();
  for (int d = tid; d < R; d += RS_THREADS)
#pragma unroll
    for (int q = 0; q < NW; q++) sh.wcnt[q][d] = 0;
  __syncthreads();
  const int64_t wbase = tile * S::TILE + (int64_t)w * WTILE;
  const uint64_t lt = lanemask_lt();
  int rk[RS_ROUNDS];  // rank of this lane's element of each round among its digit in the wave
  uint64_t kk[RS_ROUNDS];
  int32_t vv[RS_ROUNDS];
#pragma unroll
  for (int r = 0; r < RS_ROUNDS; r++) {  // all loads (keys and values) issued before the first use
    const int64_t i = wbase + r * WAVE + lane;
    kk[r] = i < n ? kin[i] : 0ull;
    vv[r] = (vin && i < n) ? vin[i] : 0;
  }
#pragma unroll
  for (int r = 0; r < RS_ROUNDS; r++) {
    const int64_t i = wbase + r * WAVE + lane;
    const bool valid = i < n;
    const int d = (int)((kk[r] >> shift) & dmask);
    const uint64_t mask = same_digit<RB>(d, valid);
    const int rank = __popcll(mask & lt);
    const int before = valid ? sh.wcnt[w][d] : 0;
    __builtin_amdgcn_wave_barrier();
    if (valid && rank == 0) sh.wcnt[w][d] = before + __popcll(mask);
    __builtin_amdgcn_wave_barrier();
    rk[r] = before + rank;
  }
  __syncthreads();
  // thread t: digits DPT t .. DPT t + DPT - 1: starts in each wave's quarter,
  // and the tile totals
  int tsum = 0;
#pragma unroll
  for (int k = 0; k < DPT; k++) {
    const int d = DPT * tid + k;
    tot[k] = 0;
#pragma unroll
    for (int q = 0; q < NW; q++) {
      const int c = sh.wcnt[q][d];
      sh.wcnt[q][d] = tot[k];
      tot[k] += c;
    }
    tsum += tot[k];
  }
  {
    const int incl = wave_incl_scan(tsum);
    if (lane == WAVE - 1) sh.wsum[w] = incl;
    __syncthreads();
    int off = 0;
    for (int q = 0; q < w; q++) off += sh.wsum[q];
    int e = off + incl - tsum;
#pragma unroll
    for (int k = 0; k < DPT; k++) {
      sh.dstart[DPT * tid + k] = e;
      e += tot[k];
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RS_ROUNDS; r++) {
    const int64_t i = wbase + r * WAVE + lane;
    if (i < n) {
      const uint64_t key = kk[r];
      const int d = (int)((key >> shift) & dmask);
      const int lp = sh.dstart[d] + sh.wcnt[w][d] + rk[r];
      sh.skey[lp] = key;
      sh.sval[lp] = vv[r];
    }
  }
  __syncthreads();
}

// The tile's elements, in digit order, to their places: a digit's run goes to
// consecutive addresses from sh.gbase[d].  GUARD: places outside [0, n) are
// skipped (they arise only after a wait of the look-back was given up, when
// the sort is reported as failed).
template <int RB, int RS_ROUNDS, bool GUARD = false>
__device__ __forceinline__ void rs_write_tile(uint64_t* kout, int32_t* vout, int64_t n,
                                              int64_t tile, int shift, uint32_t dmask,
                                              const RsTile<RB, RS_ROUNDS>& sh) {
  using S = RsTile<RB, RS_ROUNDS>;
  const int64_t base = tile * S::TILE;
  const int tn = (int)max((int64_t)0, min((int64_t)S::TILE, n - base));
  for (int j = threadIdx.x; j < tn; j += RS_THREADS) {
    const uint64_t key = sh.skey[j];
    const int d = (int)((key >> shift) & dmask);
    const int64_t o = (int64_t)sh.gbase[d] + (j - sh.dstart[d]);
    if (GUARD && (o < 0 || o >= n)) continue;
    kout[o] = key;
    if (vout) vout[o] = sh.sval[j];
  }
}

// Scatter of one tile, stable, its digits' global starts from the scanned
// per-tile histograms.
template <int RB, int RS_ROUNDS>
__global__ void __launch_bounds__(RS_THREADS)
    k_radix_scatter(const uint64_t* kin, const int32_t* vin, uint64_t* kout, int32_t* vout,
                    int64_t n, int shift, uint32_t dmask, const int32_t* hist_scan, int nblk,
                    const int64_t* n_dev, const Control* stop) {
  bookkeeping_priority();
  if (n_dev) n = min(*n_dev, n);
  if (stop && walk_aborted(stop)) n = 0;
  constexpr int R = 1 << RB;
  __shared__ RsTile<RB, RS_ROUNDS> sh;
  for (int d = threadIdx.x; d < R; d += RS_THREADS)
    sh.gbase[d] = hist_scan[(int64_t)d * nblk + blockIdx.x];
  int tot[R / RS_THREADS];
  rs_rank_tile<RB, RS_ROUNDS>(kin, vin, n, blockIdx.x, shift, dmask, sh, tot);
  rs_write_tile<RB, RS_ROUNDS>(kout, vout, n, blockIdx.x, shift, dmask, sh);
}

// ---- one launch per digit: decoupled look-back over the tiles ----
//
// The digit counts of every pass (they do not depend on the order) come from
// one histogram launch.  Each tile of a pass then takes the next tile number
// (an integer atomic: a tile waits only on tiles that started before it,
// which are resident or done), ranks its keys, publishes its digit counts and
// adds, per digit, the words of the tiles before it, newest first, up to the
// first one that holds inclusive sums (the sums of that tile and every
// earlier one); then it publishes its own inclusive sums.  The tile just
// before is read first (in the steady state it has its inclusive sums
// already), then OS_BATCH tiles at a time.  Each status word carries the
// pass's epoch (unique to the pass, so the array is never cleared) and its
// kind, and is written and read with device-scope atomic stores and loads: a
// word is seen whole or not at all, across the XCDs.  Waits are bounded: a
// tile that gives one up writes nothing and sets an error flag (the build
// then fails), and places outside the array are skipped, so the pass ends
// with wrong places but no hang and no access out of bounds.  Used for
// particle sorts of up to 2^17 keys, where it measured faster than three
// launches per digit.
constexpr int OS_BATCH = 8;           // earlier tiles' words read together
constexpr uint32_t OS_AGG = 1u;       // the tile's own digit counts
constexpr uint32_t OS_INC = 2u;       // the digit sums of the tile and every earlier one
constexpr int OS_SPIN_MAX = 1 << 20;  // polls before a wait is given up
constexpr int OS_HIST_BLOCKS = 256;   // blocks of the histogram launch (fewer atomics per counter)

__device__ __forceinline__ uint64_t os_load(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void os_store(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t os_word(uint32_t epoch, uint32_t kind, uint32_t v) {
  return ((uint64_t)epoch << 34) | ((uint64_t)kind << 32) | (uint64_t)v;
}
// kind of a status word of this pass (0: not written in this pass yet)
__device__ __forceinline__ uint32_t os_kind(uint64_t w, uint32_t epoch) {
  return (uint32_t)(w >> 34) == epoch ? (uint32_t)(w >> 32) & 3u : 0u;
}

// Digit counts of every pass: one block per chunk of keys, counts in LDS,
// then added to st->hist with integer atomics (the order does not matter).
template <int RB>
__global__ void __launch_bounds__(RS_THREADS)
    k_os_hist(const uint64_t* keys, int64_t n, int lo_bit, int passes, int last_bits,
              OsState* st, const int64_t* n_dev, const Control* stop) {
  bookkeeping_priority();
  if (n_dev) n = min(*n_dev, n);
  if (stop && walk_aborted(stop)) n = 0;
  constexpr int R = 1 << RB;
  __shared__ int h[OS_MAX_PASSES][R];
  for (int e = threadIdx.x; e < OS_MAX_PASSES * R; e += RS_THREADS) (&h[0][0])[e] = 0;
  __syncthreads();
  const int64_t per = (n + gridDim.x - 1) / gridDim.x;
  const int64_t i0 = blockIdx.x * per, i1 = min(n, i0 + per);
  for (int64_t i = i0 + threadIdx.x; i < i1; i += RS_THREADS) {
    const uint64_t k = keys[i];
    for (int p = 0; p < passes; p++) {
      const uint32_t m = p == passes - 1 ? (1u << last_bits) - 1u : (uint32_t)(R - 1);
      atomicAdd(&h[p][(int)((k >> (lo_bit + RB * p)) & m)], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < passes * R; e += RS_THREADS) {
    const int v = (&h[0][0])[e];
    if (v) atomicAdd(&st->hist[e / R][e % R], v);
  }
}

template <int RB, int RS_ROUNDS>
__global__ void __launch_bounds__(RS_THREADS)
    k_os_pass(const uint64_t* kin, const int32_t* vin, uint64_t* kout, int32_t* vout, int64_t n,
              int pass, int shift, uint32_t dmask, OsState* st, uint64_t* dword, uint32_t epoch,
              int32_t* err, const int64_t* n_dev, const Control* stop) {
  bookkeeping_priority();
  if (n_dev) n = min(*n_dev, n);
  if (stop && walk_aborted(stop)) n = 0;
  constexpr int R = 1 << RB;
  constexpr int DPT = R / RS_THREADS;
  __shared__ RsTile<RB, RS_ROUNDS> sh;
  __shared__ int tile_s, err_s;
  const int tid = threadIdx.x, lane = __lane_id();
  if (tid == 0) {
    tile_s = (int)atomicAdd(&st->tile_ctr[pass], 1u);
    err_s = 0;
  }
  // the pass's digit starts over the whole array (exclusive scan of its counts)
  int c[DPT], cs = 0;
#pragma unroll
  for (int k = 0; k < DPT; k++) {
    c[k] = st->hist[pass][DPT * tid + k];
    cs += c[k];
  }
  {
    const int incl = wave_incl_scan(cs);
    if (lane == WAVE - 1) sh.wsum[tid / WAVE] = incl;
    __syncthreads();
    int e = incl - cs;
    for (int q = 0; q < tid / WAVE; q++) e += sh.wsum[q];
#pragma unroll
    for (int k = 0; k < DPT; k++) {
      sh.gbase[DPT * tid + k] = e;
      e += c[k];
    }
  }
  const int t = tile_s;  // read after the barrier above
  int tot[DPT];
  rs_rank_tile<RB, RS_ROUNDS>(kin, vin, n, t, shift, dmask, sh, tot);
  // publish the tile's counts (tile 0: they are already its inclusive sums)
#pragma unroll
  for (int k = 0; k < DPT; k++)
    os_store(&dword[(int64_t)t * R + DPT * tid + k],
             os_word(epoch, t == 0 ? OS_INC : OS_AGG, (uint32_t)tot[k]));
  if (t > 0) {
#pragma unroll
    for (int k = 0; k < DPT; k++) {
      const int d = DPT * tid + k;
      uint32_t sum = 0;
      int spins = 0;
      // the tile just before: in the steady state it has its inclusive sums
      // already, and one word is all that needs reading
      int j = t - 1;
      for (;;) {
        const uint64_t w1 = os_load(&dword[(int64_t)j * R + d]);
        const uint32_t kind = os_kind(w1, epoch);
        if (kind != 0u) {
          sum = (uint32_t)w1;
          j = kind == OS_INC ? -1 : j - 1;
          break;
        }
        if (++spins > OS_SPIN_MAX) {
          err_s = 1;
          j = -1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      for (; j >= 0;) {
        uint64_t wv[OS_BATCH];
#pragma unroll
        for (int b = 0; b < OS_BATCH; b++)  // below tile 0: inclusive zeros
          wv[b] = j - b >= 0 ? os_load(&dword[(int64_t)(j - b) * R + d]) : os_word(epoch, OS_INC, 0);
        uint32_t part = 0;
        bool found = false, wait = false;
#pragma unroll
        for (int b = 0; b < OS_BATCH; b++) {
          if (!found && !wait) {
            const uint32_t kind = os_kind(wv[b], epoch);
            if (kind == 0u) {
              wait = true;
            } else {
              part += (uint32_t)wv[b];
              found = kind == OS_INC;
            }
          }
        }
        if (wait) {  // a tile not yet published before the first inclusive word: read again
          if (++spins > OS_SPIN_MAX) {
            err_s = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
          continue;
        }
        sum += part;
        if (found) break;
        j -= OS_BATCH;
      }
      os_store(&dword[(int64_t)t * R + d], os_word(epoch, OS_INC, sum + (uint32_t)tot[k]));
      sh.gbase[d] += (int)sum;
    }
  }
  __syncthreads();
  if (err_s) {  // this tile's offsets are unknown: nothing is written, the build fails
    if (tid == 0 && err) atomicOr(err, 1);
    return;
  }
  rs_write_tile<RB, RS_ROUNDS, true>(kout, vout, n, t, shift, dmask, sh);
}

size_t os_dword_words(int64_t n) {
  const int64_t tile = rs_tile(n);
  return (size_t)(RS_MAX_RADIX * ((n + tile - 1) / tile));
}

// Sorts on bits [lo_bit, lo_bit + bits): 9-bit digits when that saves a pass
// (63-bit Morton keys: 7 passes instead of 8), else 8-bit ones; the last
// digit is masked to the remaining bits.  With `os`, each digit is placed in
// one launch (the digit counts of all passes from one histogram launch, the
// tile offsets by look-back); otherwise per-tile histograms, their scan and a
// scatter, three to four launches per digit.
// Epochs of the single-pass sorts: one counter for every sort of the process
// (every instance of os_sort), so that no two passes that may write the same
// status array ever carry the same epoch (with a counter per instance, two
// instances sharing an array reused each other's epochs, and a tile took a
// stale word for a current one).
static std::atomic<uint32_t> os_next_epoch{0};
constexpr uint32_t OS_EPOCHS = (1u << 30) - 2;  // epochs 1 .. 2^30 - 2 (0: cleared memory)

template <int RB, int RS_ROUNDS>
static hipError_t os_sort(uint64_t* keys, int32_t* idx, uint64_t* keys_alt, int32_t* idx_alt,
                          int64_t n, int lo_bit, int bits, int passes, bool* in_alt,
                          hipStream_t st, const int64_t* n_dev, const Control* stop,
                          const OsBufs& os) {
  constexpr uint32_t EPOCHS = OS_EPOCHS;
  std::atomic<uint32_t>& next_epoch = os_next_epoch;
  const int64_t tile = RS_THREADS * RS_ROUNDS;
  const int nblk = (int)((n + tile - 1) / tile);
  const uint32_t e0 = next_epoch.fetch_add((uint32_t)passes) % EPOCHS;
  if (e0 + (uint32_t)passes > EPOCHS) {  // the epochs start again: no old word may match
    hipError_t e = hipMemsetAsync(os.dword, 0, os_dword_words(n) * 8, st);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch_fill_zero(os.state, sizeof(OsState), st);
  if (e != hipSuccess) return e;
  const int last_bits = bits - RB * (passes - 1);
  const int hb = (int)std::max<int64_t>(1, std::min<int64_t>(OS_HIST_BLOCKS, (n + 4095) / 4096));
  k_os_hist<RB><<<hb, RS_THREADS, 0, st>>>(keys, n, lo_bit, passes, last_bits, os.state, n_dev,
                                           stop);
  uint64_t *ka = keys, *kb = keys_alt;
  int32_t *va = idx, *vb = idx_alt;
  for (int pass = 0; pass < passes; pass++) {
    const int shift = lo_bit + RB * pass;
    const int db = std::min(RB, lo_bit + bits - shift);
    const uint32_t dmask = (1u << db) - 1u;
    const uint32_t epoch = 1u + (e0 + (uint32_t)pass) % EPOCHS;
    k_os_pass<RB, RS_ROUNDS><<<nblk, RS_THREADS, 0, st>>>(ka, va, kb, vb, n, pass, shift, dmask,
                                                          os.state, os.dword, epoch, os.err, n_dev,
                                                          stop);
    std::swap(ka, kb);
    std::swap(va, vb);
    *in_alt = !*in_alt;
  }
  return hipGetLastError();
}

hipError_t launch_radix_sort_bits(uint64_t* keys, int32_t* idx, uint64_t* keys_alt,
                                  int32_t* idx_alt, int64_t n, int lo_bit, int bits,
                                  int32_t* hist, int32_t* scan_tmp, bool* in_alt,
                                  hipStream_t st, const int64_t* n_dev, const Control* stop,
                                  const OsBufs* os) {
  *in_alt = false;
  if (n <= 0 || bits <= 0) return hipSuccess;
  const int64_t tile = rs_tile(n);
  const bool shortt = tile == RS_THREADS * 8;
  const int nblk = (int)((n + tile - 1) / tile);
  const int rb = (bits + 8) / 9 < (bits + 7) / 8 ? 9 : 8;
  const int passes = (bits + rb - 1) / rb;
  if (os && passes <= OS_MAX_PASSES) {
    if (rb == 9 && shortt)
      return os_sort<9, 8>(keys, idx, keys_alt, idx_alt, n, lo_bit, bits, passes, in_alt, st,
                           n_dev, stop, *os);
    if (rb == 9)
      return os_sort<9, 16>(keys, idx, keys_alt, idx_alt, n, lo_bit, bits, passes, in_alt, st,
                            n_dev, stop, *os);
    if (shortt)
      return os_sort<8, 8>(keys, idx, keys_alt, idx_alt, n, lo_bit, bits, passes, in_alt, st,
                           n_dev, stop, *os);
    return os_sort<8, 16>(keys, idx, keys_alt, idx_alt, n, lo_bit, bits, passes, in_alt, st,
                          n_dev, stop, *os);
  }
  uint64_t *ka = keys, *kb = keys_alt;
  int32_t *va = idx, *vb = idx_alt;  // both null: keys only
  for (int pass = 0; pass < passes; pass++) {
    const int shift = lo_bit + rb * pass;
    const int db = std::min(rb, lo_bit + bits - shift);
    const uint32_t dmask = (1u << db) - 1u;
    const int64_t nh = ((int64_t)1 << rb) * nblk;
    if (rb == 9 && shortt)
      k_radix_hist<9, 8><<<nblk, RS_THREADS, 0, st>>>(ka, n, shift, dmask, hist, nblk, n_dev,
                                                              stop);
    else if (rb == 9)
      k_radix_hist<9, 16><<<nblk, RS_THREADS, 0, st>>>(ka, n, shift, dmask, hist, nblk, n_dev,
                                                              stop);
    else if (shortt)
      k_radix_hist<8, 8><<<nblk, RS_THREADS, 0, st>>>(ka, n, shift, dmask, hist, nblk, n_dev,
                                                              stop);
    else
      k_radix_hist<8, 16><<<nblk, RS_THREADS, 0, st>>>(ka, n, shift, dmask, hist, nblk, n_dev,
                                                              stop);
    hipError_t e = scan_excl<int32_t>(hist, hist, nh, nullptr, scan_tmp, st);
    if (e != hipSuccess) return e;
    if (rb == 9 && shortt)
      k_radix_scatter<9, 8><<<nblk, RS_THREADS, 0, st>>>(ka, va, kb, vb, n, shift, dmask, hist,
                                                           nblk, n_dev, stop);
    else if (rb == 9)
      k_radix_scatter<9, 16><<<nblk, RS_THREADS, 0, st>>>(ka, va, kb, vb, n, shift, dmask, hist,
                                                            nblk, n_dev, stop);
    else if (shortt)
      k_radix_scatter<8, 8><<<nblk, RS_THREADS, 0, st>>>(ka, va, kb, vb, n, shift, dmask, hist,
                                                           nblk, n_dev, stop);
    else
      k_radix_scatter<8, 16><<<nblk, RS_THREADS, 0, st>>>(ka, va, kb, vb, n, shift, dmask, hist,
                                                            nblk, n_dev, stop);
    uint64_t* tk = ka;
    ka = kb;
    kb = tk;
    int32_t* tv = va;
    va = vb;
    vb = tv;
    *in_alt = !*in_alt;
  }
  return hipGetLastError();
}

hipError_t launch_radix_sort(uint64_t* keys, int32_t* idx, uint64_t* keys_alt, int32_t* idx_alt,
                             int64_t n, int32_t* hist, int32_t* scan_tmp, bool* in_alt,
                             hipStream_t st, const OsBufs* os) {
  // 7 passes of 9 bits over the 63-bit keys: the result is in (keys_alt, idx_alt)
  return launch_radix_sort_bits(keys, idx, keys_alt, idx_alt, n, 0, 63, hist, scan_tmp, in_alt,
                                st, nullptr, nullptr, os);
}

// ===================================================================
// small sets: box, keys, sort and gather in one launch
//
// For N <= FRONT_MID_MAX one block of 1024 threads does all of it: the box by a
// block reduction (min / max are exact, so the order does not matter), the
// keys as k_keys, then the same stable LSD sort with the keys and the current
// order held in LDS (12 bytes per particle): wave w owns the w-th sixteenth of
// the current order, counts its digits, the counts are scanned over waves and
// digits, and the wave places its elements in order, so equal digits keep
// their order.  Every thread reads its part of the order before any is
// written (a block barrier between), so one order buffer serves all passes.
// Replaces the 33 dependent launches of the multi-block path, which are what a
// small step costs.  Two instances:
//   * N <= FRONT_MAX: seven 9-bit digits; each thread reads its particles once
//     and keeps them in registers, and writes their records at their ranks at
//     the end (through the inverse permutation), so the only global reads are
//     one batch at the start.  The sort is bound by the ballots that rank equal
//     digits (vector instructions of one compute unit): about 4.7 us per pass
//     at 4096 particles.
//   * N <= FRONT_MID_MAX: eight 8-bit digits (the per-wave digit counts then
//     take 16 KB of LDS instead of 32, which leaves room for the keys and the
//     order of 11264 particles); the particles are read again for the records,
//     in sorted order (the set is small enough to stay in the caches).
// ===================================================================
constexpr int FRONT_THREADS = 1024;
constexpr int FRONT_WAVES = FRONT_THREADS / WAVE;

template <typename T, int MAXN, int RB, bool KEEP>
__global__ void __launch_bounds__(FRONT_THREADS)
    k_front_small(const T* __restrict__ pos, const T* __restrict__ mass, int n,
                  uint64_t* __restrict__ keys_sorted,
                  int32_t* __restrict__ perm, P4<T>* __restrict__ pts, RootInfo* root,
                  Control* ctrl) {
  constexpr int R = 1 << RB;
  constexpr int PASSES = (63 + RB - 1) / RB;
  // 64-element batches of a wave's part, at most
  constexpr int BATCH = ((MAXN + FRONT_WAVES - 1) / FRONT_WAVES + WAVE - 1) / WAVE;
  // particles per thread
  constexpr int PER = (MAXN + FRONT_THREADS - 1) / FRONT_THREADS;
  constexpr int KPER = KEEP ? PER : 1;
  __shared__ uint64_t skey[MAXN];
  __shared__ int32_t ord[MAXN];
  __shared__ int wc[FRONT_WAVES][R];
  __shared__ double bs[6][FRONT_WAVES];
  __shared__ int wsum[8];
  __shared__ RootInfo rs;
  const int tid = threadIdx.x, w = tid / WAVE, lane = __lane_id();
  // the thread's particles tid + FRONT_THREADS b, read once (all loads in
  // flight together); kept in registers until they are written in order when
  // KEEP
  T px[KPER], py[KPER], pz[KPER], pm[KPER];
  double lo[3] = {INFINITY, INFINITY, INFINITY}, hi[3] = {-INFINITY, -INFINITY, -INFINITY};
  int bad = 0;
  auto see = [&](T x, T y, T z, T m) {  // box and non-finite check
    const double v[3] = {(double)x, (double)y, (double)z};
#pragma unroll
    for (int a = 0; a < 3; a++) {
      bad |= !isfinite(v[a]);
      lo[a] = fmin(lo[a], v[a]);
      hi[a] = fmax(hi[a], v[a]);
    }
    bad |= !isfinite((double)m);
  };
  if constexpr (KEEP) {
#pragma unroll
    for (int b = 0; b < PER; b++) {
      const int i = tid + b * FRONT_THREADS;
      px[b] = py[b] = pz[b] = pm[b] = 0;
      if (i < n) {
        px[b] = pos[3 * i];
        py[b] = pos[3 * i + 1];
        pz[b] = pos[3 * i + 2];
        pm[b] = mass[i];
      }
    }
#pragma unroll
    for (int b = 0; b < PER; b++)
      if (tid + b * FRONT_THREADS < n) see(px[b], py[b], pz[b], pm[b]);
  } else {
    for (int i = tid; i < n; i += FRONT_THREADS)
      see(pos[3 * i], pos[3 * i + 1], pos[3 * i + 2], mass[i]);
  }
#pragma unroll
  for (int a = 0; a < 3; a++) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      lo[a] = fmin(lo[a], __shfl_xor(lo[a], o, WAVE));
      hi[a] = fmax(hi[a], __shfl_xor(hi[a], o, WAVE));
    }
  }
  if (lane == 0)
    for (int a = 0; a < 3; a++) {
      bs[a][w] = lo[a];
      bs[3 + a][w] = hi[a];
    }
  if (__ballot(bad) != 0ull && lane == 0) atomicOr(&ctrl->nonfinite, 1);
  __syncthreads();
  if (w < 6) {  // wave a reduces bound a over the waves (min / max are exact)
    const int a = w;
    double v = lane < FRONT_WAVES ? bs[a][lane] : (a < 3 ? INFINITY : -INFINITY);
#pragma unroll
    for (int o = FRONT_WAVES / 2; o >= 1; o >>= 1) {
      const double u = __shfl_xor(v, o, WAVE);
      v = a < 3 ? fmin(v, u) : fmax(v, u);
    }
    if (lane == 0) bs[a][0] = v;
  }
  __syncthreads();
  if (tid == 0) {
    double l[3], h[3];
    for (int a = 0; a < 3; a++) {
      l[a] = bs[a][0];
      h[a] = bs[3 + a][0];
    }
    const RootInfo r = root_cube(l, h);
    rs = r;
    *root = r;
    ctrl->root = r;
  }
  __syncthreads();
  const RootInfo r = rs;
  if constexpr (KEEP) {
#pragma unroll
    for (int b = 0; b < PER; b++) {
      const int i = tid + b * FRONT_THREADS;
      if (i < n) {
        const T v3[3] = {px[b], py[b], pz[b]};
        skey[i] = morton_key(v3, 0, r);
        ord[i] = i;
      }
    }
  } else {
    for (int i = tid; i < n; i += FRONT_THREADS) {
      const T v3[3] = {pos[3 * i], pos[3 * i + 1], pos[3 * i + 2]};
      skey[i] = morton_key(v3, 0, r);
      ord[i] = i;
    }
  }
  __syncthreads();
  // wave w's sixteenth of the order, whole batches of 64
  const int per = ((n + FRONT_WAVES - 1) / FRONT_WAVES + WAVE - 1) / WAVE * WAVE;
  const int c0 = min(n, w * per), c1 = min(n, c0 + per);
  const uint64_t lt = lanemask_lt();
  for (int pass = 0; pass < PASSES; pass++) {
    const int shift = RB * pass;
    for (int d = lane; d < R; d += WAVE) wc[w][d] = 0;
    __builtin_amdgcn_wave_barrier();
    // this lane's elements of the wave's part: index and digit (loaded first)
    int32_t sv[BATCH];
    int dg[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; b++) {
      const int i = c0 + b * WAVE + lane;
      sv[b] = i < c1 ? ord[i] : 0;
      dg[b] = i < c1 ? (int)((skey[sv[b]] >> shift) & (uint64_t)(R - 1)) : -1;
    }
    // digit counts (integer LDS atomics: the order does not matter here)
#pragma unroll
    for (int b = 0; b < BATCH; b++)
      if (dg[b] >= 0) atomicAdd(&wc[w][dg[b]], 1);
    __syncthreads();  // also: every part of the order has been read
    int incl = 0, acc = 0;
    if (tid < R) {  // digit tid: start of each wave's part within the digit
      for (int q = 0; q < FRONT_WAVES; q++) {
        const int c = wc[q][tid];
        wc[q][tid] = acc;
        acc += c;
      }
      incl = wave_incl_scan(acc);  // the first R / 64 waves: digits in order
      if (lane == WAVE - 1) wsum[w] = incl;
    }
    __syncthreads();
    if (tid < R) {
      int dstart = incl - acc;
      for (int q = 0; q < w; q++) dstart += wsum[q];
      for (int q = 0; q < FRONT_WAVES; q++) wc[q][tid] += dstart;
    }
    __syncthreads();
    // each wave places its elements in order: ranks among equal digits from
    // ballots, after the wave's running position for the digit
#pragma unroll
    for (int b = 0; b < BATCH; b++) {
      if (c0 + b * WAVE >= c1) break;  // wave-uniform
      const int d = dg[b];
      const uint64_t mask = same_digit<RB>(d, d >= 0);
      const int before = d >= 0 ? wc[w][d] : 0;
      __builtin_amdgcn_wave_barrier();
      if (d >= 0) {
        ord[before + __popcll(mask & lt)] = sv[b];
        if ((mask & lt) == 0) wc[w][d] = before + __popcll(mask);
      }
      __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
  }
  if constexpr (KEEP) {
    // the inverse of the order replaces it, and each thread writes its own
    // particles' records at their places
    int32_t ik[PER];
#pragma unroll
    for (int b = 0; b < PER; b++) {
      const int k = tid + b * FRONT_THREADS;
      ik[b] = 0;
      if (k < n) {
        const int32_t i = ord[k];
        ik[b] = i;
        perm[k] = i;
        keys_sorted[k] = skey[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < PER; b++) {
      const int k = tid + b * FRONT_THREADS;
      if (k < n) ord[ik[b]] = k;
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < PER; b++) {
      const int i = tid + b * FRONT_THREADS;
      if (i < n) {
        P4<T> q;
        q.x = px[b];
        q.y = py[b];
        q.z = pz[b];
        q.m = pm[b];
        pts[ord[i]] = q;
      }
    }
  } else {
    for (int k = tid; k < n; k += FRONT_THREADS) {
      const int32_t i = ord[k];
      perm[k] = i;
      keys_sorted[k] = skey[i];
      P4<T> q;
      q.x = pos[3 * i];
      q.y = pos[3 * i + 1];
      q.z = pos[3 * i + 2];
      q.m = mass[i];
      pts[k] = q;
    }
  }
}

template <typename T>
static void front_small_launch(const void* pos, const void* mass, int64_t n, uint64_t* keys_sorted,
                               int32_t* perm, void* pts, RootInfo* root, Control* ctrl,
                               hipStream_t st) {
  if (n <= FRONT_MAX)
    k_front_small<T, FRONT_MAX, 9, true><<<1, FRONT_THREADS, 0, st>>>(
        (const T*)pos, (const T*)mass, (int)n, keys_sorted, perm, (P4<T>*)pts, root, ctrl);
  else
    k_front_small<T, FRONT_MID_MAX, 8, false><<<1, FRONT_THREADS, 0, st>>>(
        (const T*)pos, (const T*)mass, (int)n, keys_sorted, perm, (P4<T>*)pts, root, ctrl);
}

hipError_t launch_front_small(const void* pos, const void* mass, int64_t n, int dtype,
                              uint64_t* keys_sorted, int32_t* perm, void* pts, RootInfo* root,
                              Control* ctrl, hipStream_t st) {
  if (n < 1 || n > FRONT_MID_MAX) return hipErrorInvalidValue;
  if (dtype == FMM_F64)
    front_small_launch<double>(pos, mass, n, keys_sorted, perm, pts, root, ctrl, st);
  else
    front_small_launch<float>(pos, mass, n, keys_sorted, perm, pts, root, ctrl, st);
  return hipGetLastError();
}

// ===================================================================
// gather into sorted (x, y, z, m) records
// ===================================================================
template <typename T>
__global__ void k_gather(const T* pos, const T* mass, const int32_t* perm, int64_t n, P4<T>* pts) {
  int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (k >= n) return;
  int64_t i = perm[k];
  P4<T> p;
  p.x = pos[3 * i];
  p.y = pos[3 * i + 1];
  p.z = pos[3 * i + 2];
  p.m = mass[i];
  pts[k] = p;
}

hipError_t launch_gather(const void* pos, const void* mass, const int32_t* perm, int64_t n,
                         int dtype, void* pts, hipStream_t st) {
  unsigned g = (unsigned)((n + 255) / 256);
  if (dtype == FMM_F64)
    k_gather<double><<<g, 256, 0, st>>>((const double*)pos, (const double*)mass, perm, n,
                                        (P4<double>*)pts);
  else
    k_gather<float><<<g, 256, 0, st>>>((const float*)pos, (const float*)mass, perm, n,
                                       (P4<float>*)pts);
  return hipGetLastError();
}

// ===================================================================
// octree
//
// With sorted keys, particle k's cell at level l holds more than S particles
// iff some window of S+1 consecutive particles containing k lies in one level-l
// cell, i.e. iff l <= W(k) = max over windows [j, j+S] that contain k of the
// level shared by key[j] and key[j+S].  So k's leaf is at level min(W(k)+1, 21)
// (level 0 when N <= S), and a node of level l starts at k iff k starts a
// level-l cell (the level shared with key[k-1] is < l) and l <= leaf level of k.
// Counting those starts per level and block, one scan gives every node its
// breadth-first id.
// ===================================================================
constexpr int TR_THREADS = 256;

size_t tree_blkcnt_len(int64_t n) {
  int64_t nb = (n + TR_THREADS - 1) / TR_THREADS;
  return (size_t)(2 * MAX_LEVELS * nb + 1);  // + one slot for the scan total
}

// lcp[k] = level shared with key[k-1] (-1 for k = 0); wpad[i] = level shared by
// the window starting at j = i - S (or -1 if that window does not exist).
__global__ void k_tree_lcp(const uint64_t* keys, int64_t n, int S, int8_t* lcp, int8_t* wpad,
                           int64_t wlen) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) lcp[i] = (int8_t)(i == 0 ? -1 : shared_level(keys[i - 1], keys[i]));
  if (wpad && i < wlen) {
    int64_t j = i - S;
    int8_t v = -1;
    if (j >= 0 && j + S < n) v = (int8_t)shared_level(keys[j], keys[j + S]);
    wpad[i] = v;
  }
}

// The same window maxima in one launch when the span fits a block's LDS:
// each block forms wpad[x] for x in [i0, i0 + TW_OUT + span2 - 1) (-1 past
// the end, the identity of the maximum), doubles the span in LDS up to span2,
// and writes stj[i] = max of wpad[i .. i + span2 - 1] for its outputs; it
// also writes lcp for its indices below n.
constexpr int TW_OUT = 1024;       // outputs per block
constexpr int TW_SPAN_MAX = 1024;  // largest span taken in one launch
__global__ void __launch_bounds__(256)
    k_tree_window(const uint64_t* keys, int64_t n, int S, int span2, int8_t* lcp, int8_t* stj,
                  int64_t wlen) {
  __shared__ int8_t buf[2][TW_OUT + TW_SPAN_MAX];
  const int64_t i0 = (int64_t)blockIdx.x * TW_OUT;
  int len = TW_OUT + span2 - 1;
  for (int x = threadIdx.x; x < len; x += blockDim.x) {
    const int64_t i = i0 + x;
    buf[0][x] = (int8_t)((i >= S && i < n) ? shared_level(keys[i - S], keys[i]) : -1);
  }
  for (int x = threadIdx.x; x < TW_OUT; x += blockDim.x) {
    const int64_t i = i0 + x;
    if (i < n) lcp[i] = (int8_t)(i == 0 ? -1 : shared_level(keys[i - 1], keys[i]));
  }
  __syncthreads();
  int cur = 0;
  for (int h = 1; h < span2; h *= 2) {  // spans h -> 2h
    len -= h;
    for (int x = threadIdx.x; x < len; x += blockDim.x)
      buf[cur ^ 1][x] = max(buf[cur][x], buf[cur][x + h]);
    __syncthreads();
    cur ^= 1;
  }
  for (int x = threadIdx.x; x < TW_OUT; x += blockDim.x) {
    const int64_t i = i0 + x;
    if (i < wlen) stj[i] = buf[cur][x];
  }
}

__global__ void k_tree_stmax(const int8_t* in, int8_t* out, int64_t len, int64_t half) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= len) return;
  int8_t v = in[i];
  if (i + half < len) v = max(v, in[i + half]);
  out[i] = v;
}

// leaf level per particle; per-block counts of node starts and leaf starts at
// every level (blkcnt[l * nblk + b] and blkcnt[(MAX_LEVELS + l) * nblk + b]).
__global__ void __launch_bounds__(TR_THREADS)
    k_tree_leafcount(const int8_t* lcp, const int8_t* stj, int64_t n, int S, int64_t span2,
                     int8_t* leaf_level, int64_t* blkcnt, int nblk) {
  int64_t k = blockIdx.x * (int64_t)TR_THREADS + threadIdx.x;
  int lo = 99, ll = -1;
  if (k < n) {
    int W;
    if (stj == nullptr) {
      W = -1;
    } else {
      // window starts j = k-S..k sit at wpad indices k..k+S; two overlapping
      // power-of-two spans cover them
      W = max((int)stj[k], (int)stj[k + S + 1 - span2]);
    }
    ll = min(W + 1, KEY_BITS);
    leaf_level[k] = (int8_t)ll;
    lo = lcp[k];
  }
  __shared__ int cnt[2 * MAX_LEVELS];
  if (threadIdx.x < 2 * MAX_LEVELS) cnt[threadIdx.x] = 0;
  __syncthreads();
  for (int l = 0; l < MAX_LEVELS; l++) {
    uint64_t bn = __ballot(lo < l && l <= ll);
    uint64_t bl = __ballot(lo < l && l == ll);
    if (__lane_id() == 0) {
      if (bn) atomicAdd(&cnt[l], __popcll(bn));
      if (bl) atomicAdd(&cnt[MAX_LEVELS + l], __popcll(bl));
    }
  }
  __syncthreads();
  if (threadIdx.x < 2 * MAX_LEVELS) blkcnt[(int64_t)threadIdx.x * nblk + blockIdx.x] = cnt[threadIdx.x];
}

__global__ void k_tree_levelinfo(const int64_t* scanned, int nblk, const int64_t* total,
                                 const int64_t* leafcnt_raw, Control* ctrl) {
  int l = threadIdx.x;
  if (l < MAX_LEVELS) ctrl->level_off[l] = scanned[(int64_t)l * nblk];
  if (l == MAX_LEVELS) ctrl->level_off[MAX_LEVELS] = *total;
  if (l == 0) ctrl->n_nodes = *total;
}

// leaves per level = sum over blocks of the leaf-start counts (the upper half
// of blkcnt); reduced in a fixed order by one thread per level
__global__ void __launch_bounds__(256) k_tree_leaflevels(const int64_t* blkcnt, int nblk, int64_t* out) {
  __shared__ int64_t s[256];
  const int l = blockIdx.x;  // one block per level
  int64_t v = 0;
  for (int b = threadIdx.x; b < nblk; b += 256) v += blkcnt[(int64_t)(MAX_LEVELS + l) * nblk + b];
  s[threadIdx.x] = v;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) s[threadIdx.x] += s[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[l] = s[0];
}

hipError_t launch_tree_phase1(const uint64_t* keys, int64_t n, int leaf, int8_t* lcp, int8_t* wlev,
                              int8_t* wtmp, int8_t* leaf_level, int64_t* blkcnt, void* scan_tmp,
                              Control* ctrl, hipStream_t st) {
  const int S = leaf;
  int nblk = (int)((n + TR_THREADS - 1) / TR_THREADS);
  const int8_t* stj = nullptr;
  int64_t span2 = 1;
  if ((int64_t)S < n) {
    int64_t wlen = n + S;
    int64_t want = 1;  // the span 2^J <= S + 1 < 2^(J+1)
    while (want * 2 <= (int64_t)S + 1) want *= 2;
    if (want <= TW_SPAN_MAX) {
      k_tree_window<<<(unsigned)((wlen + TW_OUT - 1) / TW_OUT), 256, 0, st>>>(keys, n, S, (int)want,
                                                                              lcp, wlev, wlen);
      span2 = want;
      stj = wlev;
    } else {
      k_tree_lcp<<<(unsigned)((wlen + 255) / 256), 256, 0, st>>>(keys, n, S, lcp, wlev, wlen);
      // sparse-table levels, one launch per doubling of the span
      int8_t *a = wlev, *b = wtmp;
      while (span2 < want) {
        k_tree_stmax<<<(unsigned)((wlen + 255) / 256), 256, 0, st>>>(a, b, wlen, span2);
        int8_t* t = a;
        a = b;
        b = t;
        span2 *= 2;
      }
      stj = a;
    }
  } else {
    k_tree_lcp<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(keys, n, S, lcp, nullptr, 0);
  }
  k_tree_leafcount<<<nblk, TR_THREADS, 0, st>>>(lcp, stj, n, S, span2, leaf_level, blkcnt, nblk);
  // leaf counts per level live in the upper half and are not scanned
  k_tree_leaflevels<<<MAX_LEVELS, 256, 0, st>>>(blkcnt, nblk, ctrl->leaves_at_level);
  int64_t total_len = (int64_t)MAX_LEVELS * nblk;
  int64_t* total = blkcnt + 2 * total_len;  // the spare slot after both halves
  hipError_t e = scan_excl<int64_t>(blkcnt, blkcnt, total_len, total, scan_tmp, st);
  if (e != hipSuccess) return e;
  k_tree_levelinfo<<<1, 64, 0, st>>>(blkcnt, nblk, total, nullptr, ctrl);
  return hipGetLastError();
}

// ---- phase 2: node records ----
__global__ void __launch_bounds__(TR_THREADS)
    k_tree_emit(const uint64_t* keys, int64_t n, const int8_t* lcp, const int8_t* leaf_level,
                const int64_t* scanned, int nblk, int64_t cap, uint8_t* level, uint64_t* prefix,
                int32_t* begin) {
  int64_t k = blockIdx.x * (int64_t)TR_THREADS + threadIdx.x;
  int lo = 99, ll = -1;
  uint64_t key = 0;
  if (k < n) {
    lo = lcp[k];
    ll = leaf_level[k];
    key = keys[k];
  }
  __shared__ int wtot[TR_THREADS / WAVE];
  const int w = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const uint64_t lt = lanemask_lt();
  for (int l = 0; l < MAX_LEVELS; l++) {
    bool f = lo < l && l <= ll;
    uint64_t b = __ballot(f);
    if (lane == 0) wtot[w] = __popcll(b);
    __syncthreads();
    int64_t id = 0;
    if (f) {
      id = scanned[(int64_t)l * nblk + blockIdx.x] + __popcll(b & lt);
      for (int j = 0; j < w; j++) id += wtot[j];
    }
    if (f && id < cap) {  // more nodes than the arrays hold: the build repeats this phase
      level[id] = (uint8_t)l;
      begin[id] = (int32_t)k;
      prefix[id] = (l == 0) ? 0ull : (key >> (3 * (KEY_BITS - l)));
    }
    __syncthreads();
  }
}

// first index in [lo, hi) with keys[i] >= v
__device__ int64_t lower_bound_u64(const uint64_t* keys, int64_t lo, int64_t hi, uint64_t v) {
  while (lo < hi) {
    int64_t mid = (lo + hi) >> 1;
    if (keys[mid] < v)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}
// first index in [lo, hi) with a[i] >= v
__device__ int64_t lower_bound_i32(const int32_t* a, int64_t lo, int64_t hi, int32_t v) {
  while (lo < hi) {
    int64_t mid = (lo + hi) >> 1;
    if (a[mid] < v)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// The node count and the levels' node ranges come from the control block
// (written by the first phase); the arrays hold `cap` nodes.  With more nodes
// than that the launch does nothing (the build repeats the phase with room);
// flags past the last node are cleared for the scan over `cap` entries.
__global__ void k_tree_nodes(const uint64_t* keys, int64_t n, int S, int64_t cap,
                             const Control* ctrl, const RootInfo* root, TreeArrays t,
                             int32_t* leaf_flag) {
  const int64_t n_nodes = ctrl->level_off[MAX_LEVELS];
  if (n_nodes > cap) return;
  int64_t id = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (id >= cap) return;
  if (id >= n_nodes) {
    leaf_flag[id] = 0;
    return;
  }
  const int64_t* lo = ctrl->level_off;  // lo[l] .. lo[l + 1]: the nodes of level l
  const int l = t.level[id];
  const int64_t k = t.begin[id];
  const uint64_t P = t.prefix[id];
  int64_t end = n;
  if (l > 0) end = lower_bound_u64(keys, k, n, (P + 1) << (3 * (KEY_BITS - l)));
  const int64_t cnt = end - k;
  t.count[id] = (int32_t)cnt;
  // parent: the level l-1 node whose range starts at or before k (last such)
  int32_t par = -1;
  if (l > 0) {
    int64_t j = lower_bound_i32(t.begin, lo[l - 1], lo[l], (int32_t)(k + 1));
    par = (int32_t)(j - 1);
  }
  t.parent[id] = par;
  const bool leaf = cnt <= S || l == KEY_BITS;
  int32_t fc = -1;
  int nc = 0;
  if (!leaf) {
    // a non-leaf has l < KEY_BITS, so lo[l + 2] is within the control block's ranges
    int64_t a = lower_bound_i32(t.begin, lo[l + 1], lo[l + 2], (int32_t)k);
    int64_t b = lower_bound_i32(t.begin, a, lo[l + 2], (int32_t)(k + cnt));
    fc = (int32_t)a;
    nc = (int)(b - a);
  }
  t.first_child[id] = fc;
  t.n_child[id] = (uint8_t)nc;
  leaf_flag[id] = leaf ? 1 : 0;
  // integer cell coordinates and geometric centre
  uint32_t qx = compact3(P >> 2), qy = compact3(P >> 1), qz = compact3(P);
  t.q[id] = ((uint64_t)qx << 42) | ((uint64_t)qy << 21) | (uint64_t)qz;
  {  // exact integer geometry in units of 1/2^22 of the root side
    const int sh = KEY_BITS - l;
    int4 g;
    g.x = (int)((2u * qx + 1u) << sh);
    g.y = (int)((2u * qy + 1u) << sh);
    g.z = (int)((2u * qz + 1u) << sh);
    g.w = (1 << sh) | (leaf ? (1 << 30) : 0);
    t.geo[id] = g;
  }
  const double w = ldexp(root->side, -l);
  const uint32_t q[3] = {qx, qy, qz};
#pragma unroll
  for (int a = 0; a < 3; a++)
    t.centre[3 * id + a] = __dadd_rn(root->lo[a], __dmul_rn((double)q[a] + 0.5, w));
}

__global__ void k_tree_leaves(const int32_t* leaf_flag, const int32_t* scan, int64_t cap,
                              const Control* ctrl, const int32_t* begin, const int32_t* count,
                              int32_t* leaves, int32_t* leaf_of, int32_t* parents) {
  const int64_t n_nodes = ctrl->level_off[MAX_LEVELS];
  if (n_nodes > cap) return;
  int64_t id = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (id >= n_nodes) return;
  if (!leaf_flag[id]) {  // non-leaf: its rank among non-leaves is id - (leaves before id)
    parents[id - scan[id]] = (int32_t)id;
    return;
  }
  leaves[scan[id]] = (int32_t)id;
  for (int32_t k = begin[id]; k < begin[id] + count[id]; k++) leaf_of[k] = (int32_t)id;
}

hipError_t launch_tree_phase2(const uint64_t* keys, int64_t n, int leaf, const int8_t* lcp,
                              const int8_t* leaf_level, const int64_t* blkcnt_scanned,
                              int64_t cap, const RootInfo* root, const TreeArrays& t,
                              int32_t* leaf_flag, int32_t* leaf_scan, int32_t* leaves,
                              int32_t* leaf_of, int32_t* parents, void* scan_tmp,
                              const Control* ctrl, hipStream_t st) {
  int nblk = (int)((n + TR_THREADS - 1) / TR_THREADS);
  k_tree_emit<<<nblk, TR_THREADS, 0, st>>>(keys, n, lcp, leaf_level, blkcnt_scanned, nblk, cap,
                                           t.level, t.prefix, t.begin);
  unsigned g = (unsigned)((cap + 255) / 256);
  k_tree_nodes<<<g, 256, 0, st>>>(keys, n, leaf, cap, ctrl, root, t, leaf_flag);
  hipError_t e = scan_excl<int32_t>(leaf_flag, leaf_scan, cap, nullptr, scan_tmp, st);
  if (e != hipSuccess) return e;
  k_tree_leaves<<<g, 256, 0, st>>>(leaf_flag, leaf_scan, cap, ctrl, t.begin, t.count, leaves,
                                   leaf_of, parents);
  return hipGetLastError();
}

}  // namespace mbg
