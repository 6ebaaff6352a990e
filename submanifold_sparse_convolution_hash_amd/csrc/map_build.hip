// Kernel-map construction for SubMConv3d on gfx950.
//
// The map is the cached, device-resident gather index of the
// trellis_sparse_mlx README ("Performance": the prepared gather index is
// built once and reused; "What's in it": the indice-map cache of the sparse
// tensor). Sites are packed injectively into one 64-bit key (the coordinate
// packing of "Running TRELLIS.2 on a Mac (3/3)", section E), inserted into an
// open-addressing hash table in HBM, and every site then finds its 27
// neighbours c + d (cross-correlation, README "Correctness"): 13 by probing
// the table, 13 by the symmetry of the map, and itself.
//
// Steps (one stream; the host waits for it twice, after the counts and at
// the end):
//   pack     coords -> keys, range validation (error flag)
//   insert   keys -> table, 64-bit compare-and-swap, linear probing; a key
//            that is already present raises the duplicate flag. When every
//            key fits in 32 bits a slot is one 64-bit word, key and row, so
//            that a probe reads both with one load
//   order    optional Morton codes + radix sort -> processing order
//   query    13 probes per site -> nbr[27][n] (tap-major): taps 0..12
//            directly, 14..26 by symmetry, 13 the site itself; and the
//            entries per tap 0..13 of each kTileRows-row tile
//   tiles    per tile of processing rows, the neighbours of each tap
//            compacted into a list of {neighbour row, row in tile}
//            (count, exclusive scan over tiles, fill)
//   readback flags + pair count: the one host wait before the lists, which
//            reports bad sites and sizes the lists (the wider tiles' counts
//            and lists follow it, read back at the final wait)
#include <rocprim/device/device_radix_sort.hpp>

#include <algorithm>
#include <cstdarg>
#include <cstring>
#include <mutex>
#include <vector>

#include "submconv_internal.h"

namespace submconv {

namespace {

thread_local std::string g_last_error;

constexpr uint64_t kEmpty = ~0ull;
constexpr uint32_t kErrRange = 1u;
constexpr uint32_t kErrDuplicate = 2u;

// MurmurHash3 64-bit finalizer (public domain, Austin Appleby): a bijective
// mixer, so distinct keys stay distinct and nearby keys scatter.
__device__ __forceinline__ uint64_t mix64(uint64_t k) {
  k ^= k >> 33;
  k *= 0xff51afd7ed558ccdull;
  k ^= k >> 33;
  k *= 0xc4ceb9fe1a85ec53ull;
  k ^= k >> 33;
  return k;
}

// key = ((b*G0 + x)*G1 + y)*G2 + z: injective for in-range sites.
__device__ __forceinline__ uint64_t pack_key(int32_t b, int32_t x, int32_t y, int32_t z, int32_t g0,
                                             int32_t g1, int32_t g2) {
  return ((static_cast<uint64_t>(b) * g0 + static_cast<uint64_t>(x)) * g1 +
          static_cast<uint64_t>(y)) *
             g2 +
         static_cast<uint64_t>(z);
}

// Spreads the low 21 bits of v so that bit i lands at bit 3i.
__device__ __forceinline__ uint64_t spread3(uint64_t v) {
  v &= 0x1fffffull;
  v = (v | (v << 32)) & 0x1f00000000ffffull;
  v = (v | (v << 16)) & 0x1f0000ff0000ffull;
  v = (v | (v << 8)) & 0x100f00f00f00f00full;
  v = (v | (v << 4)) & 0x10c30c30c30c30c3ull;
  v = (v | (v << 2)) & 0x1249249249249249ull;
  return v;
}

__global__ void k_pack(const int32_t* __restrict__ coords, int64_t n, int32_t batch, int32_t g0,
                       int32_t g1, int32_t g2, uint64_t* __restrict__ keys,
                       uint32_t* __restrict__ err, int morton_bits,
                       uint64_t* __restrict__ mcode, int32_t* __restrict__ midx) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t b = coords[4 * i + 0];
  const int32_t x = coords[4 * i + 1];
  const int32_t y = coords[4 * i + 2];
  const int32_t z = coords[4 * i + 3];
  const bool ok = b >= 0 && b < batch && x >= 0 && x < g0 && y >= 0 && y < g1 && z >= 0 && z < g2;
  if (!ok) atomicOr(err, kErrRange);
  keys[i] = ok ? pack_key(b, x, y, z, g0, g1, g2) : kEmpty;
  if (mcode) {
    uint64_t c = 0;
    if (ok)
      c = (static_cast<uint64_t>(b) << (3 * morton_bits)) |
          (spread3(static_cast<uint64_t>(x)) << 2) | (spread3(static_cast<uint64_t>(y)) << 1) |
          spread3(static_cast<uint64_t>(z));
    mcode[i] = c;
    midx[i] = static_cast<int32_t>(i);
  }
}

__global__ void k_iota(int32_t* __restrict__ v, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) v[i] = static_cast<int32_t>(i);
}

// First slot of a key: the mixed key, so that the sites of dense surfaces,
// runs of consecutive keys, do not pile up into long probe runs (keeping 8
// consecutive keys in one run of slots measured 1.4x slower on such maps).
__device__ __forceinline__ uint64_t start_slot(uint64_t key, uint64_t mask) {
  return mix64(key) & mask;
}

// COMPACT: a slot is the key (below 2^32) in the low half and the row in the
// high half, written by the one compare-and-swap; rows are below 2^31 - 1,
// so a full slot never equals the empty one. Otherwise keys and rows sit in
// two arrays.
template <bool COMPACT>
__global__ void k_insert(const uint64_t* __restrict__ keys, int64_t n, uint64_t* table,
                         int32_t* __restrict__ tvals, uint64_t mask, uint32_t* __restrict__ err) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint64_t key = keys[i];
  if (key == kEmpty) return;  // out-of-range site, already flagged
  const uint64_t want = COMPACT ? (static_cast<uint64_t>(i) << 32) | key : key;
  uint64_t h = start_slot(key, mask);
  // The table holds at most n keys in >= 2n slots, so an empty slot exists.
  while (true) {
    const unsigned long long prev = atomicCAS(reinterpret_cast<unsigned long long*>(table + h),
                                              static_cast<unsigned long long>(kEmpty),
                                              static_cast<unsigned long long>(want));
    if (prev == kEmpty) {
      if constexpr (!COMPACT) tvals[h] = static_cast<int32_t>(i);
      return;
    }
    if ((COMPACT ? (prev & 0xffffffffull) : prev) == key) {
      atomicOr(err, kErrDuplicate);
      return;
    }
    h = (h + 1) & mask;
  }
}

// Processing position of tap k (the inverse of tap_at).
__device__ __forceinline__ int pos_of(int k) {
  return k == kCenterTap ? 0 : (k < kCenterTap ? k + 1 : k);
}

// The map is symmetric: j is row i's neighbour at offset d exactly when i
// is j's neighbour at -d, and tap 26 - k has the offset of tap k negated. So
// the query probes only taps 0..12 (and fills the centre, 13): each found
// pair also gives the entry of tap 26 - k at j's processing position (inv,
// or j itself without an order), into a map whose taps 14..26 hold -1.
//
// One workgroup per (kTileRows-row tile of processing rows, tap 0..13):
// thread r probes the tap's neighbour of the tile's row r and writes
// nbr[k][t] (coalesced, tap-major). The workgroups of an XCD (blockIdx % 8)
// take one contiguous run of units, tap fastest, so that a tile's
// coordinates and the table lines its neighbours share stay in that XCD's
// L2 over its taps. Each workgroup also writes the tile's entry count at
// its tap and adds it to the tile's total (tile_tot zeroed before).
constexpr int kQueryTaps = kCenterTap + 1;
template <bool COMPACT>
__global__ __launch_bounds__(kTileRows) void k_query(
    const int32_t* __restrict__ coords, const int32_t* __restrict__ order,
    const int32_t* __restrict__ inv, int64_t n, int32_t g0, int32_t g1, int32_t g2,
    const uint64_t* __restrict__ table, const int32_t* __restrict__ tvals, uint64_t mask,
    int32_t* __restrict__ nbr, uint16_t* __restrict__ tile_cnt, int32_t* __restrict__ tile_tot,
    uint32_t units) {
  __shared__ int wcnt[kTileRows / 64];
  const uint32_t bid = blockIdx.x, xcd = bid & 7u, q = units >> 3, rem = units & 7u;
  const uint32_t u = xcd * q + (xcd < rem ? xcd : rem) + (bid >> 3);
  const uint32_t tile = u / kQueryTaps;
  const int k = static_cast<int>(u - tile * kQueryTaps);
  const int64_t t = static_cast<int64_t>(tile) * kTileRows + threadIdx.x;
  int32_t j = -1;
  if (t < n) {
    const int64_t i = order ? order[t] : t;
    if (k == kCenterTap) {
      j = static_cast<int32_t>(i);
    } else {
      const int32_t b = coords[4 * i + 0];
      const int32_t nx = coords[4 * i + 1] + (k / 9) - 1;
      const int32_t ny = coords[4 * i + 2] + ((k / 3) % 3) - 1;
      const int32_t nz = coords[4 * i + 3] + (k % 3) - 1;
      if (nx >= 0 && nx < g0 && ny >= 0 && ny < g1 && nz >= 0 && nz < g2) {
        const uint64_t key = pack_key(b, nx, ny, nz, g0, g1, g2);
        uint64_t h = start_slot(key, mask);
        while (true) {
          const uint64_t s = table[h];
          if (s == kEmpty) break;
          if ((COMPACT ? (s & 0xffffffffull) : s) == key) {
            j = COMPACT ? static_cast<int32_t>(s >> 32) : tvals[h];
            break;
          }
          h = (h + 1) & mask;
        }
      }
      if (j >= 0)
        nbr[static_cast<int64_t>(kTaps3 - 1 - k) * n + (inv ? inv[j] : j)] = static_cast<int32_t>(i);
    }
    nbr[static_cast<int64_t>(k) * n + t] = j;
  }
  const uint64_t m = __ballot(j >= 0);
  if ((threadIdx.x & 63) == 0) wcnt[threadIdx.x >> 6] = __popcll(m);
  __syncthreads();
  if (threadIdx.x == 0) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kTileRows / 64; ++w) c += wcnt[w];
    tile_cnt[static_cast<int64_t>(tile) * kTaps3 + pos_of(k)] = static_cast<uint16_t>(c);
    atomicAdd(tile_tot + tile, c);
  }
}

// Clears a build's scratch in one launch: the hash table's slots (all ones),
// a run of words to zero (flags, pair count, groups, tile totals) and a run
// of map entries to -1 (the taps the query fills by symmetry).
__global__ void k_init(uint64_t* __restrict__ table, int64_t cap, uint32_t* __restrict__ zero,
                       int64_t n_zero, int32_t* __restrict__ none, int64_t n_none) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (int64_t i = i0; i < cap; i += stride) table[i] = kEmpty;
  for (int64_t i = i0; i < n_zero; i += stride) zero[i] = 0u;
  for (int64_t i = i0; i < n_none; i += stride) none[i] = -1;
}

// inv[order[t]] = t: the processing position of each row.
__global__ void k_invert(const int32_t* __restrict__ order, int64_t n, int32_t* __restrict__ inv) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t < n) inv[order[t]] = static_cast<int32_t>(t);
}

// The sums of one tile set after its counts, in one launch with a fixed
// summation order and no atomics. Blocks 0..26: the groups of kGroupRows
// entries at processing position p, over the tiles (the work of the weight
// gradient's positions). Block 27: the tiles' list offsets, an exclusive scan
// of the tile totals whose entry n_tiles holds all entries, and the active
// pairs in 64 bits when asked for (the int32 offsets are checked against it).
__global__ __launch_bounds__(1024) void k_tile_sums(const int32_t* __restrict__ tile_tot,
                                                    const uint16_t* __restrict__ tile_cnt,
                                                    int64_t n_tiles, int32_t* __restrict__ tile_off,
                                                    unsigned long long* __restrict__ pairs,
                                                    unsigned long long* __restrict__ groups) {
  __shared__ unsigned long long part[1024];
  const int tid = threadIdx.x;
  if (blockIdx.x < kTaps3) {
    const int p = blockIdx.x;
    unsigned long long s = 0;
    for (int64_t t = tid; t < n_tiles; t += 1024)
      s += (tile_cnt[t * kTaps3 + p] + kGroupRows - 1) / kGroupRows;
    part[tid] = s;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
      if (tid < w) part[tid] += part[tid + w];
      __syncthreads();
    }
    if (tid == 0) groups[p] = part[0];
    return;
  }
  // thread tid owns the tiles [lo, hi): their sum, a scan of the 1024 sums,
  // then the running offsets
  const int64_t per = (n_tiles + 1023) / 1024;
  const int64_t lo = std::min<int64_t>(tid * per, n_tiles);
  const int64_t hi = std::min<int64_t>(lo + per, n_tiles);
  unsigned long long s = 0;
  for (int64_t t = lo; t < hi; ++t) s += static_cast<unsigned long long>(tile_tot[t]);
  part[tid] = s;
  __syncthreads();
  for (int w = 1; w < 1024; w <<= 1) {  // inclusive scan
    const unsigned long long v = tid >= w ? part[tid - w] : 0ull;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  unsigned long long run = part[tid] - s;
  for (int64_t t = lo; t < hi; ++t) {
    tile_off[t] = static_cast<int32_t>(run);
    run += static_cast<unsigned long long>(tile_tot[t]);
  }
  if (tid == 1023) {
    tile_off[n_tiles] = static_cast<int32_t>(part[1023]);
    if (pairs) *pairs = part[1023];
  }
}

// Sorted-key builder (the packing + sort + search lookup of "Running
// TRELLIS.2 on a Mac (3/3)", section E): an independent second way to the
// same map. skeys/srows are the packed keys and their rows sorted by key.
__global__ void k_sorted_dups(const uint64_t* __restrict__ skeys, int64_t n, uint64_t none,
                              uint32_t* __restrict__ err) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t > 0 && t < n && skeys[t] != none && skeys[t] == skeys[t - 1]) atomicOr(err, kErrDuplicate);
}

// One thread per (tap k, processing row t), t fastest: nbr[k][t] by a binary
// search (lower bound) of the neighbour's key among the sorted keys.
__global__ void k_query_sorted(const int32_t* __restrict__ coords, const int32_t* __restrict__ order,
                               int64_t n, int32_t g0, int32_t g1, int32_t g2,
                               const uint64_t* __restrict__ skeys, const int32_t* __restrict__ srows,
                               int32_t* __restrict__ nbr) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx < n * kTaps3) {
    const int k = static_cast<int>(idx / n);
    const int64_t t = idx - static_cast<int64_t>(k) * n;
    const int64_t i = order ? order[t] : t;
    const int32_t b = coords[4 * i + 0];
    const int32_t nx = coords[4 * i + 1] + (k / 9) - 1;
    const int32_t ny = coords[4 * i + 2] + ((k / 3) % 3) - 1;
    const int32_t nz = coords[4 * i + 3] + (k % 3) - 1;
    int32_t j = -1;
    if (k == kCenterTap) {
      j = static_cast<int32_t>(i);
    } else if (nx >= 0 && nx < g0 && ny >= 0 && ny < g1 && nz >= 0 && nz < g2) {
      const uint64_t key = pack_key(b, nx, ny, nz, g0, g1, g2);
      int64_t lo = 0, hi = n;
      while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (skeys[mid] < key) lo = mid + 1; else hi = mid;
      }
      if (lo < n && skeys[lo] == key) j = srows[lo];
    }
    nbr[idx] = j;
  }
}

// Per tile of tr <= TR processing rows: entries of taps k_lo..26 per
// processing position (wave ballots over 64-row chunks; a block has TR
// rounded up to 64 threads), added to the tile's total.
template <int TR>
__global__ __launch_bounds__((TR + 63) / 64 * 64) void k_tile_count(
    const int32_t* __restrict__ nbr, int64_t n, int tr, int k_lo, uint16_t* __restrict__ tile_cnt,
    int32_t* __restrict__ tile_tot) {
  constexpr int NWV = (TR + 63) / 64;
  __shared__ int cnt[NWV][kTaps3];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * tr + threadIdx.x;
  const bool valid = static_cast<int>(threadIdx.x) < tr && t < n;
  for (int k = k_lo; k < kTaps3; ++k) {
    const uint64_t m = __ballot(valid && nbr[static_cast<int64_t>(k) * n + t] >= 0);
    if (lane == 0) cnt[w][k] = __popcll(m);
  }
  __syncthreads();
  if (threadIdx.x < kTaps3 && tap_at(threadIdx.x) >= k_lo) {
    const int k = tap_at(threadIdx.x);
    int c = 0;
    for (int ww = 0; ww < NWV; ++ww) c += cnt[ww][k];
    tile_cnt[static_cast<int64_t>(blockIdx.x) * kTaps3 + threadIdx.x] = static_cast<uint16_t>(c);
  }
  if (threadIdx.x == 0) {
    int tot = 0;
    for (int k = k_lo; k < kTaps3; ++k)
      for (int ww = 0; ww < NWV; ++ww) tot += cnt[ww][k];
    atomicAdd(tile_tot + blockIdx.x, tot);
  }
}

// Writes the tile's entries {neighbour's caller row, row in tile}, ordered by
// processing position, then row.
template <int TR>
__global__ __launch_bounds__((TR + 63) / 64 * 64) void k_tile_fill(
    const int32_t* __restrict__ nbr, int64_t n, int tr, const int32_t* __restrict__ tile_off,
    int2* __restrict__ ent) {
  constexpr int NWV = (TR + 63) / 64;
  __shared__ uint64_t masks[kTaps3][NWV];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * tr + threadIdx.x;
  const bool valid = static_cast<int>(threadIdx.x) < tr && t < n;
  int32_t v[kTaps3];
  for (int k = 0; k < kTaps3; ++k) {
    v[k] = valid ? nbr[static_cast<int64_t>(k) * n + t] : -1;
    const uint64_t m = __ballot(v[k] >= 0);
    if (lane == 0) masks[k][w] = m;
  }
  __syncthreads();
  // one more entry {-1, -1} after all lists: the target of masked loads
  if (blockIdx.x == 0 && threadIdx.x == 0) ent[tile_off[gridDim.x]] = make_int2(-1, -1);
  const uint64_t below = (1ull << lane) - 1ull;
  int64_t base = tile_off[blockIdx.x];
  for (int p = 0; p < kTaps3; ++p) {
    const int k = tap_at(p);
    int before = 0, total = 0;
    for (int ww = 0; ww < NWV; ++ww) {
      const int c = __popcll(masks[k][ww]);
      before += ww < w ? c : 0;
      total += c;
    }
    const uint64_t m = masks[k][w];
    if ((m >> lane) & 1ull) {
      int2 e;
      e.x = v[k];
      e.y = static_cast<int>(threadIdx.x);
      ent[base + before + __popcll(m & below)] = e;
    }
    base += total;
  }
}

__global__ void k_export(const int32_t* __restrict__ nbr, const int32_t* __restrict__ order,
                         int64_t n, int32_t* __restrict__ kmap) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n * kTaps3) return;
  const int64_t k = idx / n;
  const int64_t t = idx - k * n;
  const int64_t i = order ? order[t] : t;
  kmap[i * kTaps3 + k] = nbr[idx];
}

__global__ void k_order_out(const int32_t* __restrict__ order, int64_t n, int32_t* __restrict__ out) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t < n) out[t] = order ? order[t] : static_cast<int32_t>(t);
}

// The order of the wide tiles in each XCD's run (one workgroup per XCD). A
// forward with one workgroup per CU deals the tiles of XCD x, [x tpx,
// (x+1) tpx), to its wpx workgroups by run position: workgroup j takes
// positions j, j + wpx, ... A tile's cost is the steps the forward gives it
// (the centre's, then one per 32 entries of each other position, the
// off-centre part padded to a multiple of 4) plus about an epilogue's worth.
// The costliest tiles go first (ties: the lower tile), each to the workgroup
// with the least cost so far that still has a position (ties: the lower
// workgroup), so that the workgroups finish together; tiles stay in their
// XCD's run, whose neighbouring rows share its L2. Runs of more than
// kWalkMax tiles (many units per workgroup, which even out by themselves),
// and more than 64 workgroups per XCD (one wave places the tiles), keep
// their order.
constexpr int kWalkMax = 256;
__global__ __launch_bounds__(kWalkMax) void k_tile_walk(const uint16_t* __restrict__ cnt,
                                                         int64_t nt, int64_t tpx, int wpx,
                                                         int32_t* __restrict__ walk) {
  constexpr int kGroup = 32, kCentre = kTileRowsWide / kGroup;
  constexpr int kRound = (4 - kCentre % 4) % 4, kEpilogue = 3;
  __shared__ uint32_t key[kWalkMax];  // cost << 16 | (0xffff - index): descending = costliest, lowest
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * tpx;
  const int64_t hi = lo + tpx < nt ? lo + tpx : nt;
  if (hi <= lo) return;
  const int count = static_cast<int>(hi - lo);
  const int tid = threadIdx.x;
  if (count > kWalkMax || wpx > 64) {
    for (int64_t i = lo + tid; i < hi; i += blockDim.x) walk[i] = static_cast<int32_t>(i);
    return;
  }
  uint32_t k = 0;
  if (tid < count) {
    int f = kCentre;
    for (int p = 1; p < kTaps3; ++p) f += (cnt[(lo + tid) * kTaps3 + p] + kGroup - 1) / kGroup;
    const int off = f - kCentre - kRound > 0 ? f - kCentre - kRound : 0;
    const int steps = kCentre + kRound + ((off + 3) & ~3);
    const uint32_t c = static_cast<uint32_t>((steps > 8 ? steps : 8) + kEpilogue);
    k = (c << 16) | static_cast<uint32_t>(0xffff - tid);
  }
  key[tid] = k;
  __syncthreads();
  // bitonic sort, descending
  for (int size = 2; size <= kWalkMax; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int partner = tid ^ stride;
      if (partner > tid) {
        const uint32_t a = key[tid], b = key[partner];
        const bool desc = (tid & size) == 0;
        if (desc ? a < b : a > b) {
          key[tid] = b;
          key[partner] = a;
        }
      }
      __syncthreads();
    }
  }
  // greedy placement by the first wave: lane j is workgroup j
  if (tid >= 64) return;
  const int w = wpx < count ? wpx : count;
  int64_t load = 0;
  int used = 0;
  for (int i = 0; i < count; ++i) {
    const uint32_t ki = key[i];
    const int tile = 0xffff - static_cast<int>(ki & 0xffff);
    const int c = static_cast<int>(ki >> 16);
    const bool open = tid < w && tid + used * w < count;
    // the least-loaded open workgroup, the lowest on a tie (loads stay far below 2^40)
    int64_t v = open ? (load << 6) | tid : INT64_MAX;
    for (int sh = 1; sh < 64; sh <<= 1) {
      const int64_t o = __shfl_xor(v, sh, 64);
      v = o < v ? o : v;
    }
    if (open && (v & 63) == tid) {
      walk[lo + tid + static_cast<int64_t>(used) * w] = static_cast<int32_t>(lo + tile);
      load += c;
      ++used;
    }
  }
}

inline unsigned grid_for(int64_t n, int block) {
  return static_cast<unsigned>((n + block - 1) / block);
}

int bits_for(int64_t extent) {  // smallest b with 2^b >= extent (at least 1)
  int b = 1;
  while ((int64_t{1} << b) < extent) ++b;
  return b;
}

// A build's scratch (keys, hash table, sort space, counts) stays with its
// device after the build, up to kKeepScratch bytes, for the next build: its
// allocation and release otherwise take about as much host time as a small
// build's kernels. A build holds its device's lease from taking the scratch
// to its last wait for the stream, so builds on one device take turns.
constexpr size_t kKeepScratch = size_t{256} << 20;
constexpr int kScratchDevices = 64;
struct KeptScratch {
  std::mutex mu;
  void* p = nullptr;
  size_t bytes = 0;
};
KeptScratch g_kept[kScratchDevices];

class ScratchLease {
 public:
  explicit ScratchLease(int device)
      : kept_(device >= 0 && device < kScratchDevices ? &g_kept[device] : nullptr) {
    if (kept_) lock_ = std::unique_lock<std::mutex>(kept_->mu);
  }
  ScratchLease(const ScratchLease&) = delete;
  ScratchLease& operator=(const ScratchLease&) = delete;
  // at least `bytes` of device memory, the kept scratch when it is as large
  hipError_t take(size_t bytes, void** out) {
    if (kept_ && kept_->p && kept_->bytes >= bytes) {
      p_ = kept_->p;
      bytes_ = kept_->bytes;
      kept_->p = nullptr;
      kept_->bytes = 0;
    } else {
      if (kept_ && kept_->p) {
        (void)hipFree(kept_->p);
        kept_->p = nullptr;
        kept_->bytes = 0;
      }
      const hipError_t e = hipMalloc(&p_, bytes);
      if (e != hipSuccess) {
        p_ = nullptr;
        return e;
      }
      bytes_ = bytes;
    }
    *out = p_;
    return hipSuccess;
  }
  // the stream no longer uses the scratch when this runs
  ~ScratchLease() {
    if (!p_) return;
    if (kept_ && bytes_ <= kKeepScratch) {
      kept_->p = p_;
      kept_->bytes = bytes_;
    } else {
      (void)hipFree(p_);
    }
  }

 private:
  KeptScratch* kept_;
  std::unique_lock<std::mutex> lock_;
  void* p_ = nullptr;
  size_t bytes_ = 0;
};

// Sparse map: fewer than one kGroupRows-entry group per off-centre position
// of a 256-row tile on average, so that a tile's step count barely grows
// with its rows.
bool sparse_map(int64_t n, int64_t pairs) {
  return (pairs - n) * kTileRows < int64_t{kGroupRows} * (kTaps3 - 1) * n;
}

// Rows of the wider tiles a sparse map would take: when tiles of up to 288
// rows need fewer rounds of one tile per compute unit than 256-row ones, the
// fewest rows that fit the tiles into those rounds; otherwise 0 (none).
int wide_tile_rows(int64_t n, int cus) {
  if (n <= 0 || cus <= 0) return 0;
  const int64_t r256 = ((n + kTileRows - 1) / kTileRows + cus - 1) / cus;
  const int64_t r288 = ((n + kTileRowsWide - 1) / kTileRowsWide + cus - 1) / cus;
  if (r288 >= r256) return 0;
  const int64_t slots = r288 * cus;
  const int tr = static_cast<int>(std::min<int64_t>((n + slots - 1) / slots, kTileRowsWide));
  return tr > kTileRows ? tr : 0;
}

// Hands out 256-byte aligned pieces of one allocation: a first pass with no
// base sizes it, a second pass over the same requests gives the pointers.
struct Carve {
  char* base = nullptr;
  size_t used = 0;
  template <class T>
  T* take(size_t count) {
    const size_t at = (used + 255) & ~size_t{255};
    used = at + sizeof(T) * (count > 0 ? count : 1);
    return base ? reinterpret_cast<T*>(base + at) : nullptr;
  }
};

}  // namespace

int set_error(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

void clear_error() { g_last_error.clear(); }

const char* last_error_cstr() { return g_last_error.c_str(); }

}  // namespace submconv

using namespace submconv;

extern "C" int submconv_build_map(const int32_t* coords, int64_t n, int32_t batch,
                                  const int32_t grid[3], uint32_t flags, hipStream_t stream,
                                  submconv_map_t* out_map) {
  clear_error();
  if (!out_map) return set_error(SUBMCONV_ERR_INVALID_ARG, "out_map is NULL");
  *out_map = nullptr;
  if (!grid) return set_error(SUBMCONV_ERR_INVALID_ARG, "grid is NULL");
  if (n < 0) return set_error(SUBMCONV_ERR_INVALID_ARG, "n = %lld is negative", (long long)n);
  if (n > 0 && !coords) return set_error(SUBMCONV_ERR_INVALID_ARG, "coords is NULL");
  if (batch < 1) return set_error(SUBMCONV_ERR_INVALID_ARG, "batch = %d < 1", batch);
  if (flags & ~(SUBMCONV_FLAG_MORTON | SUBMCONV_FLAG_SORTED_KEYS | SUBMCONV_FLAG_TILES_256 |
                SUBMCONV_FLAG_TILES_288 | SUBMCONV_FLAG_STAGED | SUBMCONV_FLAG_NO_STAGED))
    return set_error(SUBMCONV_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if ((flags & SUBMCONV_FLAG_TILES_256) && (flags & SUBMCONV_FLAG_TILES_288))
    return set_error(SUBMCONV_ERR_INVALID_ARG, "flags ask for two tile sizes");
  if ((flags & SUBMCONV_FLAG_STAGED) && (flags & SUBMCONV_FLAG_NO_STAGED))
    return set_error(SUBMCONV_ERR_INVALID_ARG, "flags ask for and against the staged plan");
  for (int a = 0; a < 3; ++a)
    if (grid[a] < 1) return set_error(SUBMCONV_ERR_INVALID_ARG, "grid[%d] = %d < 1", a, grid[a]);
  if (n > INT32_MAX - 1)
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "n = %lld exceeds int32 row indices",
                     (long long)n);
  // the packed key must not overflow 63 bits: batch * G0 * G1 * G2 < 2^63
  {
    unsigned __int128 v = static_cast<unsigned __int128>(batch);
    for (int a = 0; a < 3; ++a) v *= static_cast<unsigned __int128>(grid[a]);
    if (v >= (static_cast<unsigned __int128>(1) << 63))
      return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "batch*grid volume exceeds 2^63");
  }
  const bool morton = (flags & SUBMCONV_FLAG_MORTON) != 0;
  const bool sorted_keys = (flags & SUBMCONV_FLAG_SORTED_KEYS) != 0;
  int mbits = 0;
  if (morton) {
    mbits = bits_for(std::max(grid[0], std::max(grid[1], grid[2])));
    const int bbits = batch > 1 ? bits_for(batch) : 0;
    if (mbits > 21 || 3 * mbits + bbits > 64)
      return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "grid too large for a 64-bit Morton code");
  }

  Map m;
  SUBMCONV_HIP_CHECK(hipGetDevice(&m.device));
  m.n = n;
  m.batch = batch;
  for (int a = 0; a < 3; ++a) m.grid[a] = grid[a];
  m.flags = flags;
  if (n == 0) {
    *out_map = new submconv_map_s{m};
    return SUBMCONV_OK;
  }
  {
    // the forwards on this map that take W as it is stage it here
    const int st = ensure_weight_stage(m.device);
    if (st != SUBMCONV_OK) return st;
  }

  int64_t cap = 64;
  while (cap < 2 * n) cap <<= 1;
  const uint64_t mask = static_cast<uint64_t>(cap - 1);
  // one-word slots when every packed key is below 2^32
  bool compact = true;
  {
    uint64_t v = static_cast<uint64_t>(batch);
    for (int a = 0; a < 3 && compact; ++a) {
      v *= static_cast<uint64_t>(grid[a]);  // < 2^63 (checked above)
      compact = v <= (uint64_t{1} << 32);
    }
  }

  // tile sets: 256-row tiles always; wider ones when asked for, or (unless
  // 256 rows are asked for) when the map turns out sparse and they save a
  // round of tiles
  int cus = 256;
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, m.device);
  const int wide_cand = (flags & SUBMCONV_FLAG_TILES_288)   ? kTileRowsWide
                        : (flags & SUBMCONV_FLAG_TILES_256) ? 0
                                                            : wide_tile_rows(n, cus);
  const int64_t nt_base = (n + kTileRows - 1) / kTileRows;
  const int64_t nt_wide = wide_cand > 0 ? (n + wide_cand - 1) / wide_cand : 0;
  // tiles of the staged plan, unless it is ruled out
  const int64_t nt_stage =
      (flags & SUBMCONV_FLAG_NO_STAGED) ? 0 : (n + kStageUnitRows - 1) / kStageUnitRows;

  // library scratch sizes, asked for before anything is allocated
  size_t ksort_bytes = 0, msort_bytes = 0;
  const int bbits = batch > 1 ? bits_for(batch) : 0;
  const unsigned end_bit = static_cast<unsigned>(3 * mbits + bbits);
  auto check_size = [&](hipError_t e) -> int {
    if (e != hipSuccess)
      return set_error(SUBMCONV_ERR_HIP, "scratch size query failed: %s", hipGetErrorString(e));
    return SUBMCONV_OK;
  };
  if (sorted_keys)
    if (const int st = check_size(rocprim::radix_sort_pairs(
            nullptr, ksort_bytes, static_cast<const uint64_t*>(nullptr), static_cast<uint64_t*>(nullptr),
            static_cast<const int32_t*>(nullptr), static_cast<int32_t*>(nullptr),
            static_cast<size_t>(n), 0u, 64u, stream));
        st != SUBMCONV_OK)
      return st;
  if (morton)
    if (const int st = check_size(rocprim::radix_sort_pairs(
            nullptr, msort_bytes, static_cast<const uint64_t*>(nullptr), static_cast<uint64_t*>(nullptr),
            static_cast<const int32_t*>(nullptr), static_cast<int32_t*>(nullptr),
            static_cast<size_t>(n), 0u, end_bit, stream));
        st != SUBMCONV_OK)
      return st;

  // the build's temporaries, in one allocation freed on return
  struct Temps {
    uint64_t *keys, *tkeys, *skeys, *mcode_in, *mcode_out;
    int32_t *tvals, *srows, *rows_in, *midx, *inv, *tile_tot, *tile_tot_wide;
    void *small, *ksort, *msort;
  } t{};
  StagedTemps stp;
  stp.n_tiles = nt_stage;
  auto temps = [&](Carve& c) {
    t.keys = c.take<uint64_t>(n);
    if (sorted_keys) {
      t.skeys = c.take<uint64_t>(n);
      t.srows = c.take<int32_t>(n);
      t.rows_in = c.take<int32_t>(n);
      t.ksort = c.take<char>(ksort_bytes);
    } else {
      t.tkeys = c.take<uint64_t>(cap);
      if (!compact) t.tvals = c.take<int32_t>(cap);
    }
    if (morton) {
      t.mcode_in = c.take<uint64_t>(n);
      t.mcode_out = c.take<uint64_t>(n);
      t.midx = c.take<int32_t>(n);
      if (!sorted_keys) t.inv = c.take<int32_t>(n);
      t.msort = c.take<char>(msort_bytes);
    }
    // zeroed together, at the end: flags and sums, and the tile totals
    t.small = c.take<char>(512);
    t.tile_tot = c.take<int32_t>(nt_base + 1);
    t.tile_tot_wide = c.take<int32_t>(nt_wide + 1);
    if (nt_stage > 0) {
      stp.tile_units = c.take<int4>(kStageMaxUnitsPerTile * nt_stage);
      stp.tile_nu = c.take<int32_t>(nt_stage);
      stp.tile_ns = c.take<int32_t>(nt_stage);
      stp.unit_off = c.take<int64_t>(nt_stage);
      stp.staged_off = c.take<int64_t>(nt_stage);
      stp.totals = c.take<int64_t>(2);
    }
  };
  // what the map keeps, but the lists (sized once the pairs are counted)
  Tiles base, wide;
  int32_t* nbr = nullptr;
  int32_t* order = nullptr;
  auto kept = [&](Carve& c) {
    nbr = c.take<int32_t>(kTaps3 * n);
    if (morton) order = c.take<int32_t>(n);
    base.cnt = c.take<uint16_t>(kTaps3 * nt_base);
    base.off = c.take<int32_t>(nt_base + 1);
    if (nt_wide > 0) {
      wide.cnt = c.take<uint16_t>(kTaps3 * nt_wide);
      wide.off = c.take<int32_t>(nt_wide + 1);
      wide.walk = c.take<int32_t>(nt_wide);
    }
  };

  ScratchLease lease(m.device);  // released after the waits below
  void* tmp = nullptr;
  void* mem = nullptr;
  void* ent_mem = nullptr;
  void* staged_mem = nullptr;
  auto fail = [&](int status) {
    (void)hipStreamSynchronize(stream);
    if (mem) (void)hipFree(mem);
    if (ent_mem) (void)hipFree(ent_mem);
    if (staged_mem) (void)hipFree(staged_mem);
    return status;
  };
#define BUILD_CHECK(expr)                                                                 \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess)                                                                 \
      return fail(set_error(e_ == hipErrorOutOfMemory ? SUBMCONV_ERR_OUT_OF_MEMORY        \
                                                      : SUBMCONV_ERR_HIP,                 \
                            "%s failed: %s", #expr, hipGetErrorString(e_)));             \
  } while (0)

  {
    Carve c;
    temps(c);
    BUILD_CHECK(lease.take(c.used, &tmp));
    c = Carve{static_cast<char*>(tmp), 0};
    temps(c);
  }
  {
    Carve c;
    kept(c);
    BUILD_CHECK(hipMalloc(&mem, c.used));
    c = Carve{static_cast<char*>(mem), 0};
    kept(c);
  }
  uint32_t* err = static_cast<uint32_t*>(t.small);
  unsigned long long* pairs = reinterpret_cast<unsigned long long*>(static_cast<char*>(t.small) + 8);

  const int B = 256;
  {
    const int64_t n_table = sorted_keys ? 0 : cap;
    const int64_t n_zero =
        (reinterpret_cast<char*>(t.tile_tot_wide + nt_wide + 1) - static_cast<char*>(t.small)) / 4;
    // the hash query fills taps 14..26 by symmetry
    const int64_t n_none = sorted_keys ? 0 : (kTaps3 - kQueryTaps) * n;
    const int64_t most = std::max(n_table, std::max(n_zero, n_none));
    k_init<<<static_cast<unsigned>(std::min<int64_t>((most + B - 1) / B, 2048)), B, 0, stream>>>(
        t.tkeys, n_table, static_cast<uint32_t*>(t.small), n_zero, nbr + kQueryTaps * n, n_none);
    BUILD_CHECK(hipGetLastError());
  }
  k_pack<<<grid_for(n, B), B, 0, stream>>>(coords, n, batch, grid[0], grid[1], grid[2], t.keys, err,
                                           mbits, t.mcode_in, t.midx);
  BUILD_CHECK(hipGetLastError());
  if (sorted_keys) {
    // rows 0..n-1 as the sort's values; out-of-range sites carry the empty
    // key, which sorts last and matches no query
    k_iota<<<grid_for(n, B), B, 0, stream>>>(t.rows_in, n);
    BUILD_CHECK(hipGetLastError());
    BUILD_CHECK(rocprim::radix_sort_pairs(t.ksort, ksort_bytes, static_cast<const uint64_t*>(t.keys),
                                          t.skeys, static_cast<const int32_t*>(t.rows_in), t.srows,
                                          static_cast<size_t>(n), 0u, 64u, stream));
    k_sorted_dups<<<grid_for(n, B), B, 0, stream>>>(t.skeys, n, kEmpty, err);
  } else if (compact) {
    k_insert<true><<<grid_for(n, B), B, 0, stream>>>(t.keys, n, t.tkeys, nullptr, mask, err);
  } else {
    k_insert<false><<<grid_for(n, B), B, 0, stream>>>(t.keys, n, t.tkeys, t.tvals, mask, err);
  }
  BUILD_CHECK(hipGetLastError());
  if (morton) {
    BUILD_CHECK(rocprim::radix_sort_pairs(t.msort, msort_bytes,
                                          static_cast<const uint64_t*>(t.mcode_in), t.mcode_out,
                                          static_cast<const int32_t*>(t.midx), order,
                                          static_cast<size_t>(n), 0u, end_bit, stream));
    if (!sorted_keys) {
      k_invert<<<grid_for(n, B), B, 0, stream>>>(order, n, t.inv);
      BUILD_CHECK(hipGetLastError());
    }
  }
  if (sorted_keys) {
    k_query_sorted<<<grid_for(n * kTaps3, B), B, 0, stream>>>(coords, order, n, grid[0], grid[1],
                                                              grid[2], t.skeys, t.srows, nbr);
  } else {
    // the query also counts the 256-row tiles' entries of taps 0..13
    const uint32_t units = static_cast<uint32_t>(nt_base * kQueryTaps);
    if (compact)
      k_query<true><<<units, kTileRows, 0, stream>>>(coords, order, t.inv, n, grid[0], grid[1],
                                                     grid[2], t.tkeys, nullptr, mask, nbr, base.cnt,
                                                     t.tile_tot, units);
    else
      k_query<false><<<units, kTileRows, 0, stream>>>(coords, order, t.inv, n, grid[0], grid[1],
                                                      grid[2], t.tkeys, t.tvals, mask, nbr, base.cnt,
                                                      t.tile_tot, units);
  }
  BUILD_CHECK(hipGetLastError());

  // per-tile compacted lists of tr-row tiles: counts (into zeroed totals),
  // list offsets and groups per position; for the 256-row tiles also the
  // active pairs (the same for every tile size)
  unsigned long long* groups_wide =
      reinterpret_cast<unsigned long long*>(static_cast<char*>(t.small) + 256);
  // (the hash query counts taps 0..13 of the 256-row tiles itself: k_lo)
  auto count_tiles = [&](int tr, Tiles& T, int32_t* tot, int k_lo, bool total,
                         unsigned long long* groups) -> int {
    const int64_t n_tiles = (n + tr - 1) / tr;
    T.rows = tr;
    T.n = n_tiles;
    if (tr > kTileRows)
      k_tile_count<kTileRowsWide><<<static_cast<unsigned>(n_tiles), (kTileRowsWide + 63) / 64 * 64,
                                    0, stream>>>(nbr, n, tr, k_lo, T.cnt, tot);
    else
      k_tile_count<kTileRows><<<static_cast<unsigned>(n_tiles), kTileRows, 0, stream>>>(
          nbr, n, tr, k_lo, T.cnt, tot);
    BUILD_CHECK(hipGetLastError());
    k_tile_sums<<<kTaps3 + 1, 1024, 0, stream>>>(tot, T.cnt, n_tiles, T.off, total ? pairs : nullptr,
                                                 groups);
    BUILD_CHECK(hipGetLastError());
    return SUBMCONV_OK;
  };
  // the lists themselves, and the entry {-1, -1} after them
  auto fill_tiles = [&](Tiles& T) -> int {
    if (T.rows > kTileRows)
      k_tile_fill<kTileRowsWide><<<static_cast<unsigned>(T.n), (kTileRowsWide + 63) / 64 * 64, 0,
                                   stream>>>(nbr, n, T.rows, T.off, T.ent);
    else
      k_tile_fill<kTileRows><<<static_cast<unsigned>(T.n), kTileRows, 0, stream>>>(nbr, n, T.rows,
                                                                                  T.off, T.ent);
    BUILD_CHECK(hipGetLastError());
    return SUBMCONV_OK;
  };
  // the one host wait before the lists: flags, active pairs, groups
  uint64_t host_small[2 + kTaps3] = {};
  if (const int st = count_tiles(kTileRows, base, t.tile_tot, sorted_keys ? 0 : kQueryTaps, true, pairs + 1); st != SUBMCONV_OK)
    return st;
  BUILD_CHECK(hipMemcpyAsync(host_small, t.small, sizeof(host_small), hipMemcpyDeviceToHost, stream));
  BUILD_CHECK(hipStreamSynchronize(stream));
  for (int q = 0; q < kTaps3; ++q) base.pos_groups[q] = static_cast<int64_t>(host_small[2 + q]);
  const uint32_t eflags = static_cast<uint32_t>(host_small[0]);
  if (eflags & kErrRange)
    return fail(set_error(SUBMCONV_ERR_COORD_OUT_OF_RANGE,
                          "a site lies outside [0,%d) x [0,%d) x [0,%d) x [0,%d)", batch, grid[0],
                          grid[1], grid[2]));
  if (eflags & kErrDuplicate)
    return fail(set_error(SUBMCONV_ERR_DUPLICATE_COORD, "a site occurs more than once"));
  m.active_pairs = static_cast<int64_t>(host_small[1]);
  if (m.active_pairs >= INT32_MAX)
    return fail(set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "too many active pairs for int32 offsets"));
  const bool use_wide =
      wide_cand > 0 && ((flags & SUBMCONV_FLAG_TILES_288) || sparse_map(n, m.active_pairs));
  if (!use_wide) wide = Tiles{};  // its counts and offsets go unused
  // the wider tiles' counts run while the lists are allocated
  if (use_wide)
    if (const int st = count_tiles(wide_cand, wide, t.tile_tot_wide, 0, false, groups_wide);
        st != SUBMCONV_OK)
      return st;
  {
    const size_t lists = (use_wide ? 2 : 1) * static_cast<size_t>(m.active_pairs + 1);
    BUILD_CHECK(hipMalloc(&ent_mem, sizeof(int2) * lists));
    base.ent = static_cast<int2*>(ent_mem);
    if (use_wide) wide.ent = base.ent + (m.active_pairs + 1);
  }
  if (const int st = fill_tiles(base); st != SUBMCONV_OK) return st;
  uint64_t host_groups[kTaps3] = {};
  if (use_wide) {
    if (const int st = fill_tiles(wide); st != SUBMCONV_OK) return st;
    // the walk order for a forward with one workgroup per CU (cus / 8 per XCD)
    k_tile_walk<<<8, kWalkMax, 0, stream>>>(wide.cnt, wide.n, (wide.n + 7) / 8,
                                            std::max(1, cus / 8), wide.walk);
    BUILD_CHECK(hipGetLastError());
    BUILD_CHECK(hipMemcpyAsync(host_groups, groups_wide, sizeof(host_groups), hipMemcpyDeviceToHost,
                               stream));
  }
  // the staged plan of a dense map (or of any map, when asked for): its
  // units are counted before the wait, and written after it
  const bool want_staged =
      nt_stage > 0 && ((flags & SUBMCONV_FLAG_STAGED) ||
                       m.active_pairs >= int64_t{kStageMinPairsPerRow} * n);
  int64_t host_staged[2] = {0, 0};
  if (want_staged) {
    if (const int st = staged_count(nbr, n, stp, stream); st != SUBMCONV_OK) return fail(st);
    BUILD_CHECK(hipMemcpyAsync(host_staged, stp.totals, sizeof(host_staged), hipMemcpyDeviceToHost,
                               stream));
  }
  // the forward may run on another stream: the map is complete on return
  BUILD_CHECK(hipStreamSynchronize(stream));
  if (use_wide)
    for (int q = 0; q < kTaps3; ++q) wide.pos_groups[q] = static_cast<int64_t>(host_groups[q]);
  Staged staged;
  // (the kernel's staged-row offsets are 32-bit)
  if (want_staged && host_staged[0] > 0 && host_staged[1] < INT32_MAX) {
    staged.n_units = host_staged[0];
    staged.n_rows = host_staged[1];
    auto parts = [&](Carve& c) {
      staged.units = c.take<int4>(staged.n_units);
      staged.rows = c.take<int32_t>(staged.n_rows);
      staged.idx = c.take<uint16_t>(kTaps3 * staged_idx_stride(n));
    };
    Carve c;
    parts(c);
    BUILD_CHECK(hipMalloc(&staged_mem, c.used));
    c = Carve{static_cast<char*>(staged_mem), 0};
    parts(c);
    if (const int st = staged_fill(nbr, n, stp, staged, stream); st != SUBMCONV_OK) return fail(st);
    BUILD_CHECK(hipStreamSynchronize(stream));
  }
  m.mem = mem;
  m.ent_mem = ent_mem;
  m.nbr = nbr;
  m.order = order;
  m.tiles = base;
  m.wide = wide;
  m.wide_always = (flags & SUBMCONV_FLAG_TILES_288) != 0;
  m.staged_mem = staged_mem;
  m.staged = staged;
  *out_map = new submconv_map_s{m};
  return SUBMCONV_OK;
#undef BUILD_CHECK
}

extern "C" int submconv_release_scratch(void) {
  clear_error();
  int dev = -1;
  SUBMCONV_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kScratchDevices) return SUBMCONV_OK;
  KeptScratch& k = g_kept[dev];
  std::lock_guard<std::mutex> lock(k.mu);  // waits for a build in progress on the device
  if (k.p) {
    const hipError_t e = hipFree(k.p);
    k.p = nullptr;
    k.bytes = 0;
    SUBMCONV_HIP_CHECK(e);
  }
  return SUBMCONV_OK;
}

extern "C" int64_t submconv_map_num_rows(submconv_map_t map) {
  if (!map) return set_error(SUBMCONV_ERR_INVALID_ARG, "map is NULL");
  return map->m.n;
}

extern "C" int32_t submconv_map_tile_rows(submconv_map_t map) {
  if (!map) return set_error(SUBMCONV_ERR_INVALID_ARG, "map is NULL");
  return map->m.wide.n > 0 ? map->m.wide.rows : map->m.tiles.rows;
}

extern "C" int64_t submconv_map_active_pairs(submconv_map_t map, int32_t ksize) {
  if (!map) return set_error(SUBMCONV_ERR_INVALID_ARG, "map is NULL");
  if (ksize == 1) return map->m.n;
  if (ksize == 3) return map->m.active_pairs;
  return set_error(SUBMCONV_ERR_INVALID_ARG, "ksize = %d is not 1 or 3", ksize);
}

extern "C" int submconv_map_staged(submconv_map_t map, int64_t out[2]) {
  clear_error();
  if (!map || !out) return set_error(SUBMCONV_ERR_INVALID_ARG, "map or out is NULL");
  out[0] = map->m.staged.n_units;
  out[1] = map->m.staged.n_rows;
  return SUBMCONV_OK;
}

extern "C" int submconv_map_export(submconv_map_t map, int32_t* kmap, hipStream_t stream) {
  clear_error();
  if (!map) return set_error(SUBMCONV_ERR_INVALID_ARG, "map is NULL");
  const Map& m = map->m;
  if (m.n == 0) return SUBMCONV_OK;
  if (!kmap) return set_error(SUBMCONV_ERR_INVALID_ARG, "kmap is NULL");
  const int B = 256;
  k_export<<<grid_for(m.n * kTaps3, B), B, 0, stream>>>(m.nbr, m.order, m.n, kmap);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

extern "C" int submconv_map_order(submconv_map_t map, int32_t* order, hipStream_t stream) {
  clear_error();
  if (!map) return set_error(SUBMCONV_ERR_INVALID_ARG, "map is NULL");
  const Map& m = map->m;
  if (m.n == 0) return SUBMCONV_OK;
  if (!order) return set_error(SUBMCONV_ERR_INVALID_ARG, "order is NULL");
  const int B = 256;
  k_order_out<<<grid_for(m.n, B), B, 0, stream>>>(m.order, m.n, order);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

extern "C" int submconv_map_free(submconv_map_t map) {
  clear_error();
  if (!map) return SUBMCONV_OK;
  int status = SUBMCONV_OK;
  if (map->m.mem && hipFree(map->m.mem) != hipSuccess)
    status = set_error(SUBMCONV_ERR_HIP, "hipFree of the map failed");
  if (map->m.ent_mem && hipFree(map->m.ent_mem) != hipSuccess)
    status = set_error(SUBMCONV_ERR_HIP, "hipFree of the tile lists failed");
  if (map->m.staged_mem && hipFree(map->m.staged_mem) != hipSuccess)
    status = set_error(SUBMCONV_ERR_HIP, "hipFree of the staged plan failed");
  delete map;
  return status;
}

extern "C" const char* submconv_status_string(int status) {
  switch (status) {
    case SUBMCONV_OK: return "ok";
    case SUBMCONV_ERR_INVALID_ARG: return "invalid argument";
    case SUBMCONV_ERR_COORD_OUT_OF_RANGE: return "coordinate out of range";
    case SUBMCONV_ERR_DUPLICATE_COORD: return "duplicate coordinate";
    case SUBMCONV_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case SUBMCONV_ERR_HIP: return "HIP runtime error";
    case SUBMCONV_ERR_OUT_OF_MEMORY: return "out of device memory";
    default: return "unknown status";
  }
}

extern "C" const char* submconv_last_error(void) { return submconv::last_error_cstr(); }

extern "C" int submconv_abi_version(void) { return SUBMCONV_ABI_VERSION; }
