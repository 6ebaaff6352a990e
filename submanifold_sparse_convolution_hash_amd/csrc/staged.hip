// Staged SubMConv3d forward for dense maps with few channels, on gfx950.
//
// On a dense map (a surface, where a row has ~21 of its 27 neighbours) the
// compacted-list kernel gathers every (row, tap) pair from L2: each feature
// row ~21 times. Here a unit of up to 128 consecutive output rows first
// copies the distinct neighbour rows of all its taps into LDS (about 2-3.5x
// the unit's rows under Morton or raster order), and every tap reads its
// operands from there; the fp32 accumulators stay in registers, as in an
// implicit GEMM over the unit's rows (the fused [N, 27 Cin] x [27 Cin, Cout]
// product of the trellis_sparse_mlx README, "Performance"), with a zero row
// standing in for absent neighbours (the README's "Correctness" sentinel).
//
// Each of the 4 waves takes every fourth tap (k = w, w + 4, ...) for all rows
// and columns of the unit, so a tap's weights are loaded once per unit and
// wave; the four partial sums of a row are added in wave order at the end
// (((p0 + p1) + p2) + p3), so a row's result depends on neither its unit nor
// the map's row order.
//
// The plan (which rows form a unit, which rows it stages, and where each
// neighbour sits among them) is built with the map: per tile of 128 rows the
// neighbours are deduplicated in an LDS hash table, and a tile whose
// distinct neighbours exceed kStageCap is halved until its parts fit.
#include <climits>

#include "submconv_internal.h"

namespace submconv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------

constexpr int kPlanThreads = 256;
// The hash holds at most kStageCap + kPlanThreads distinct rows (below), so
// that twice the cap never fills.
constexpr int kHashSlots = 2 * kStageCap;
// Parts are halved with the left half rounded down to even rows, so a right
// half can exceed half by 2: parts of a 128-row tile reach at most 10 rows
// at depth 4, and a tile has at most 16 units.
constexpr int kMaxUnitsPerTile = kStageMaxUnitsPerTile;
static_assert(kStageCap + kPlanThreads < kHashSlots, "the hash never fills");
static_assert(kTaps3 * kStageMinRows <= kStageCap, "a smallest unit always fits");
static_assert(kStageUnitRows / 16 + 2 <= kStageMinRows, "depth-4 parts always fit");
static_assert(kStageCap < kStageNone, "staged rows fit 16 bits");

// Knuth's multiplicative hash of a row index, 10 bits
__device__ __forceinline__ int hash_slot(int32_t key) {
  return static_cast<int>((static_cast<uint32_t>(key) * 2654435761u) >> 22);
}
static_assert(kHashSlots == 1 << 10, "hash bits");

// A part's neighbour rows usually lie within a narrow range of row indices
// (in raster order a few planes of the grid, in Morton order most often
// within 64k rows): a bitmap over [kmin, kmin + kBitmapBits) then lists them
// distinct and sorted at once, a row's rank among them being the set bits
// before its own. Wider parts take the hash table and a rank count.
constexpr int kBitmapBits = 1 << 16;
constexpr int kBitmapWords = kBitmapBits / 32;

struct PlanLds {
  int32_t H[kHashSlots];   // hash table of neighbour rows, -1 empty
  alignas(16) int32_t L[kStageCap];  // the distinct rows
  uint16_t V[kHashSlots];  // slot -> position in the sorted rows
  int count;               // rows inserted into H
  int wsum[kPlanThreads / 64];
  uint32_t BM[kBitmapWords];   // bit i: row kmin + i is a neighbour
  uint16_t WP[kBitmapWords];   // set bits in the words before each word
  int kmin, kmax;
};

__device__ __forceinline__ int find_slot(const PlanLds& P, int32_t key) {
  int h = hash_slot(key);
  while (P.H[h] != key) h = (h + 1) & (kHashSlots - 1);
  return h;
}

// A part's candidates, the neighbour rows of its rows over all taps (-1
// none): thread tid holds candidates c = tid + 256 q, of tap c / rows and
// row c % rows, all requested before any is used.
constexpr int kCandsPerThread = (kTaps3 * kStageUnitRows + kPlanThreads - 1) / kPlanThreads;
__device__ __forceinline__ void load_cands(const int32_t* __restrict__ nbr, int64_t n, int64_t t0,
                                           int rows, int32_t (&key)[kCandsPerThread]) {
  const int cands = kTaps3 * rows;
#pragma unroll
  for (int q = 0; q < kCandsPerThread; ++q) {
    const int c = static_cast<int>(threadIdx.x) + kPlanThreads * q;
    const int k = c / rows;
    key[q] = c < cands ? nbr[static_cast<int64_t>(k) * n + t0 + (c - k * rows)] : -1;
  }
}

// The distinct rows among the workgroup's candidates, inserted into P.H:
// returns their number U (the same in every thread) when it is at most
// kStageCap, with the rows listed in P.L[0..U); otherwise some number above
// kStageCap. A thread inserts a row only while fewer than kStageCap + 1 are
// in, so at most kStageCap + kPlanThreads ever are.
__device__ int collect(const int32_t (&key)[kCandsPerThread], PlanLds& P) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < kHashSlots; i += kPlanThreads) P.H[i] = -1;
  if (tid == 0) P.count = 0;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kCandsPerThread; ++q) {
    if (key[q] >= 0 &&
        __hip_atomic_load(&P.count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) <= kStageCap) {
      int h = hash_slot(key[q]);
      while (true) {
        const int prev = atomicCAS(&P.H[h], -1, key[q]);
        if (prev == -1) {
          atomicAdd(&P.count, 1);
          break;
        }
        if (prev == key[q]) break;
        h = (h + 1) & (kHashSlots - 1);
      }
    }
  }
  __syncthreads();
  const int U = P.count;
  if (U > kStageCap) return U;
  constexpr int SPT = kHashSlots / kPlanThreads;
  int cnt = 0;
  for (int i = 0; i < SPT; ++i) cnt += P.H[i * kPlanThreads + tid] >= 0 ? 1 : 0;
  int incl = cnt;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) P.wsum[w] = incl;
  __syncthreads();
  int pos = incl - cnt;
  for (int ww = 0; ww < w; ++ww) pos += P.wsum[ww];
  for (int i = 0; i < SPT; ++i) {
    const int32_t k = P.H[i * kPlanThreads + tid];
    if (k >= 0) P.L[pos++] = k;
  }
  __syncthreads();
  return U;
}

// The bitmap path: the range of the candidates, and when it is narrower than
// kBitmapBits, their bitmap and its word prefix; returns the number of
// distinct rows, or -1 for a wider range (the same in every thread).
__device__ int collect_bitmap(const int32_t (&key)[kCandsPerThread], PlanLds& P) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int mn = INT_MAX, mx = -1;
#pragma unroll
  for (int q = 0; q < kCandsPerThread; ++q)
    if (key[q] >= 0) {
      mn = key[q] < mn ? key[q] : mn;
      mx = key[q] > mx ? key[q] : mx;
    }
  for (int off = 32; off > 0; off >>= 1) {
    const int a = __shfl_xor(mn, off, 64), b = __shfl_xor(mx, off, 64);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
  if (tid == 0) {
    P.kmin = INT_MAX;
    P.kmax = -1;
  }
  __syncthreads();
  if (lane == 0) {
    atomicMin(&P.kmin, mn);
    atomicMax(&P.kmax, mx);
  }
  __syncthreads();
  mn = P.kmin;
  mx = P.kmax;
  if (mx < 0) return 0;
  if (mx - mn >= kBitmapBits) return -1;
  // only the words the range covers
  const int nw = ((mx - mn) >> 5) + 1;
  for (int i = tid; i < nw; i += kPlanThreads) P.BM[i] = 0;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kCandsPerThread; ++q)
    if (key[q] >= 0) {
      const int b = key[q] - mn;
      atomicOr(&P.BM[b >> 5], 1u << (b & 31));
    }
  __syncthreads();
  // thread tid's words tid*W .. tid*W + W - 1 (of the nw in use), then a
  // block scan of their counts
  const int wpt = (nw + kPlanThreads - 1) / kPlanThreads;
  int cnt = 0;
  for (int i = 0; i < wpt; ++i) {
    const int wd = tid * wpt + i;
    cnt += wd < nw ? __popc(P.BM[wd]) : 0;
  }
  int incl = cnt;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) P.wsum[w] = incl;
  __syncthreads();
  int pos = incl - cnt, total = 0;
  for (int ww = 0; ww < kPlanThreads / 64; ++ww) {
    pos += ww < w ? P.wsum[ww] : 0;
    total += P.wsum[ww];
  }
  for (int i = 0; i < wpt; ++i) {
    const int wd = tid * wpt + i;
    if (wd < nw) {
      P.WP[wd] = static_cast<uint16_t>(pos);
      pos += __popc(P.BM[wd]);
    }
  }
  if (tid == 0) P.count = nw;  // (the words in use, for bitmap_rows)
  __syncthreads();
  return total;
}

// rank of candidate row r among the bitmap's rows
__device__ __forceinline__ int bitmap_rank(const PlanLds& P, int32_t r) {
  const int b = r - P.kmin;
  return P.WP[b >> 5] + __popc(P.BM[b >> 5] & ((1u << (b & 31)) - 1u));
}

// the bitmap's rows in order to srows
__device__ void bitmap_rows(const PlanLds& P, int32_t* __restrict__ srows) {
  const int mn = P.kmin, nw = P.count;
  for (int wd = threadIdx.x; wd < nw; wd += kPlanThreads) {
    uint32_t m = P.BM[wd];
    int pos = P.WP[wd];
    while (m) {
      const int b = __ffs(m) - 1;
      m &= m - 1;
      srows[pos++] = mn + 32 * wd + b;
    }
  }
}

// Places each distinct row at its rank among them (rows ascending): V[slot]
// = rank for the row's hash slot, and the sorted rows go to srows. The rows
// are distinct, so a row's rank is the number of smaller ones.
__device__ void rank_rows(PlanLds& P, int U, int32_t* __restrict__ srows) {
  for (int i = threadIdx.x; i < U; i += kPlanThreads) {
    const int32_t r = P.L[i];
    int rank = 0;
    for (int j = 0; j < U; ++j) rank += P.L[j] < r ? 1 : 0;
    P.V[find_slot(P, r)] = static_cast<uint16_t>(rank);
    srows[rank] = r;
  }
  __syncthreads();
}

// Per tile of kStageUnitRows processing rows: its units, found depth first
// (left half first, so in row order) by halving every part whose distinct
// neighbours exceed kStageCap, down to kStageMinRows rows.
__global__ __launch_bounds__(kPlanThreads) void k_stage_count(const int32_t* __restrict__ nbr,
                                                              int64_t n, int4* __restrict__ tile_units,
                                                              int32_t* __restrict__ tile_nu,
                                                              int32_t* __restrict__ tile_ns) {
  __shared__ PlanLds P;
  const int64_t tile = blockIdx.x;
  const int64_t t0 = tile * kStageUnitRows;
  const int trows = static_cast<int>(n - t0 < kStageUnitRows ? n - t0 : kStageUnitRows);
  // part (lvl, idx): bit lvl-1-l of idx says which half was taken at split l
  int lvl = 0, idx = 0, nu = 0, ns = 0;
  while (true) {
    int a = 0, b = trows;
    for (int l = lvl - 1; l >= 0; --l) {
      const int mid = a + (((b - a) / 2) & ~1);  // units start on even rows
      if ((idx >> l) & 1)
        a = mid;
      else
        b = mid;
    }
    int32_t key[kCandsPerThread];
    load_cands(nbr, n, t0 + a, b - a, key);
    int U = collect_bitmap(key, P);
    if (U < 0) U = collect(key, P);
    if (U <= kStageCap || b - a <= kStageMinRows) {
      if (threadIdx.x == 0) tile_units[tile * kMaxUnitsPerTile + nu] = make_int4(a, b - a, U, 0);
      ++nu;
      ns += U;
      while (lvl > 0 && (idx & 1)) {
        idx >>= 1;
        --lvl;
      }
      if (lvl == 0) break;
      ++idx;
    } else {
      ++lvl;
      idx <<= 1;
    }
  }
  if (threadIdx.x == 0) {
    tile_nu[tile] = nu;
    tile_ns[tile] = ns;
  }
}

// Exclusive scans of the tiles' unit and staged-row counts (one workgroup),
// and the totals.
__global__ __launch_bounds__(1024) void k_stage_scan(const int32_t* __restrict__ tile_nu,
                                                     const int32_t* __restrict__ tile_ns,
                                                     int64_t n_tiles, int64_t* __restrict__ unit_off,
                                                     int64_t* __restrict__ staged_off,
                                                     int64_t* __restrict__ totals) {
  __shared__ long long wu[16], ws[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  long long cu = 0, cs = 0;
  for (int64_t base = 0; base < n_tiles; base += 1024) {
    const int64_t i = base + tid;
    const long long u = i < n_tiles ? tile_nu[i] : 0, s = i < n_tiles ? tile_ns[i] : 0;
    long long iu = u, is = s;
    for (int off = 1; off < 64; off <<= 1) {
      const long long yu = __shfl_up(iu, off, 64), ys = __shfl_up(is, off, 64);
      if (lane >= off) {
        iu += yu;
        is += ys;
      }
    }
    if (lane == 63) {
      wu[w] = iu;
      ws[w] = is;
    }
    __syncthreads();
    long long bu = 0, bs = 0, tu = 0, ts = 0;
    for (int ww = 0; ww < 16; ++ww) {
      bu += ww < w ? wu[ww] : 0;
      bs += ww < w ? ws[ww] : 0;
      tu += wu[ww];
      ts += ws[ww];
    }
    if (i < n_tiles) {
      unit_off[i] = cu + bu + iu - u;
      staged_off[i] = cs + bs + is - s;
    }
    cu += tu;
    cs += ts;
    __syncthreads();
  }
  if (tid == 0) {
    totals[0] = cu;
    totals[1] = cs;
  }
}

// Writes the plan of each tile's units: the unit, its staged rows (sorted)
// and each neighbour's place among them.
__global__ __launch_bounds__(kPlanThreads) void k_stage_fill(
    const int32_t* __restrict__ nbr, int64_t n, const int4* __restrict__ tile_units,
    const int32_t* __restrict__ tile_nu, const int64_t* __restrict__ unit_off,
    const int64_t* __restrict__ staged_off, int4* __restrict__ units, int32_t* __restrict__ srows,
    uint16_t* __restrict__ sidx, int64_t stride) {
  __shared__ PlanLds P;
  const int64_t tile = blockIdx.x;
  const int64_t t0 = tile * kStageUnitRows;
  const int nu = tile_nu[tile];
  const int64_t uo = unit_off[tile];
  int64_t so = staged_off[tile];
  for (int j = 0; j < nu; ++j) {
    const int4 d = tile_units[tile * kMaxUnitsPerTile + j];  // row in tile, rows, staged rows
    const int64_t u0 = t0 + d.x;
    int32_t key[kCandsPerThread];
    load_cands(nbr, n, u0, d.y, key);
    int U = collect_bitmap(key, P);
    const bool bitmap = U >= 0;
    if (bitmap) {
      bitmap_rows(P, srows + so);
    } else {
      U = collect(key, P);
      rank_rows(P, U, srows + so);
    }
    const int cands = kTaps3 * d.y;
#pragma unroll
    for (int q = 0; q < kCandsPerThread; ++q) {
      const int c = static_cast<int>(threadIdx.x) + kPlanThreads * q;
      if (c < cands) {
        const int k = c / d.y;
        sidx[static_cast<int64_t>(k) * stride + u0 + (c - k * d.y)] =
            key[q] < 0 ? kStageNone
                       : (bitmap ? bitmap_rank(P, key[q]) : P.V[find_slot(P, key[q])]);
      }
    }
    if (threadIdx.x == 0)
      units[uo + j] = make_int4(static_cast<int>(u0), d.y, static_cast<int>(so), U);
    so += U;
    __syncthreads();  // the next unit clears the hash
  }
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ half8 bload_h8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <bool IS_BF16>
__device__ __forceinline__ _Float16 round16(float v) {
  if constexpr (IS_BF16)
    return __builtin_bit_cast(_Float16, static_cast<__bf16>(v));  // round to nearest even
  else
    return static_cast<_Float16>(v);  // round to nearest even
}

template <int CIN, int COUT>
struct CfgSt {
  static constexpr int NT = 256;             // 4 waves
  static constexpr int KS = CIN / 16;        // MFMA K steps per row
  static constexpr int RC = CIN / 8;         // 16-byte chunks per row
  static constexpr int NCB = COUT / 32;      // 32-column blocks
  static constexpr int RED = 3 * 4 * 64;            // float4s of one row block's partial sums
  // staged rows and the zero row, in chunks; with 32 output columns the
  // space also takes the four row blocks' partial sums at once (the zero row
  // is written again with every unit)
  static constexpr int STG0 = (kStageCap + 1) * RC;
  static constexpr int STG = NCB > 1 || STG0 > 4 * RED ? STG0 : 4 * RED;
  static constexpr int MAXJ = kStageCap * RC / NT;  // staging loads per thread
  static constexpr int IW = kTaps3 * kStageUnitRows / 2;  // the staged-row table, in words
  static constexpr int IJ = (IW + NT - 1) / NT;           // its loads per thread
  static constexpr int SPT = kStageCap / NT;              // staged-row indices per thread
  static constexpr int RPR = STG / RED < 4 ? STG / RED : 4;  // row blocks per round
  // k_fwd_staged (32 output columns): a wave keeps all 7 of its taps'
  // weights in registers for all its units (at 64 input channels that spills
  // a few registers, saved and restored outside the multiply loop: still
  // faster than reloading 108 KiB of weights per unit); with fewer resident
  // taps the others are loaded two taps ahead of their multiply.
  // k_fwd_staged_c64 (64 output columns) loads every tap's weights two taps
  // ahead.
  static constexpr int NRES = 7;
  static_assert((CIN == 32 || CIN == 64) && (COUT == 32 || COUT == 64) && CIN * COUT < 64 * 64,
                "shape");
  static_assert(kStageCap % NT == 0 && IW % 64 == 0 && (kStageCap * RC) % NT == 0, "layout");
};

typedef __attribute__((address_space(3))) void lds_void;

// Chunk c of staged row s sits at s*RC + (c ^ swz(s)): rows that follow each
// other fill the 16 bank groups of a 256-byte line, so that the 16 lanes of
// a read pass that take consecutive staged rows hit distinct banks.
template <int RC>
__device__ __forceinline__ int swz(int s) {
  return (s / (16 / RC)) & (RC - 1);
}

// Persistent: the workgroups of XCD x (blockIdx % 8) walk that XCD's
// contiguous run of units, neighbouring units (which stage many of the same
// rows) sharing its L2; each takes every wpx-th unit of the run. While a
// unit multiplies, the next unit's descriptor and staged-row indices are on
// their way, so that staging a unit waits for one memory round trip (its
// feature rows and table) rather than three.
template <int CIN, int COUT, bool IS_BF16>
__global__ __launch_bounds__(256, 2) void k_fwd_staged(
    const int4* __restrict__ units, int n_units, int per_xcd, int wpx,
    const int32_t* __restrict__ srows, const uint32_t* __restrict__ sidx2, int64_t istride2,
    const int32_t* __restrict__ order, int64_t n, const _Float16* __restrict__ feats,
    const _Float16* __restrict__ wp, const float* __restrict__ bias, _Float16* __restrict__ out) {
  using C = CfgSt<CIN, COUT>;
  constexpr int KS = C::KS, RC = C::RC, NCB = C::NCB, NRES = C::NRES;
  static_assert(NCB == 1, "32 output columns (64: k_fwd_staged_c64)");
  __shared__ half8 stg[C::STG];
  __shared__ uint32_t itab[C::IW];      // [27][128] staged rows of the unit's rows, two per word
  __shared__ int32_t sbuf[kStageCap];   // the unit's staged rows (caller rows)

  const int bid = blockIdx.x;
  const int xcd = bid & 7, j0 = bid >> 3;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ntaps = (kTaps3 - w + 3) / 4;  // this wave's taps k = w + 4 i
  // taps past the wave's last load tap 26 again and go unused, so that no
  // load sits in a branch (the compiler's waits for loads would otherwise
  // assume the fewest in flight after the branch)
  auto tap = [&](int i) { return w + 4 * i < kTaps3 ? w + 4 * i : kTaps3 - 1; };

  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wp, static_cast<uint32_t>(kTaps3 * CIN * COUT * 2));
  // the weights of tap k, columns 32 cb.. (1 KiB per K step, in fragment order)
  auto load_a = [&](int k, int cb, half8 (&A)[KS]) {
    const uint32_t base = static_cast<uint32_t>(((k * NCB + cb) * KS) * 1024 + lane * 16);
#pragma unroll
    for (int st = 0; st < KS; ++st) A[st] = bload_h8(rw, base + st * 1024);
  };
  // v_mfma_f32_32x32x16: A = weights (lane: column lane%32, K steps st of
  // lane half h = lane/32: channels h CIN/2 + 8 st + 0..7), B = staged rows
  // (lane: row lane%32 of the block, the same channels); D: lane holds row
  // lane%32 and columns 8 a + 4 h + b in register 4 a + b.
  // AR: the resident taps' weights; AT: a two-slot ring for the others
  half8 AR[NRES > 0 ? NRES : 1][KS];
  half8 AT[2][KS];
#pragma unroll
  for (int i = 0; i < NRES; ++i) load_a(tap(i), 0, AR[i]);

  // a unit's descriptor, staged-row indices (to sbuf) and table words (to
  // itab): requested by fetch_*, stored by put_*
  auto unit_of = [&](int ju) { return ju < per_xcd ? xcd * per_xcd + ju : n_units; };
  auto fetch_rows = [&](const int4& d, int (&SR)[C::SPT]) {
#pragma unroll
    for (int q = 0; q < C::SPT; ++q) {
      const int sr = tid + C::NT * q;
      SR[q] = sr < d.w ? srows[d.z + sr] : -1;
    }
  };
  auto put_rows = [&](const int (&SR)[C::SPT]) {
#pragma unroll
    for (int q = 0; q < C::SPT; ++q) sbuf[tid + C::NT * q] = SR[q];
  };

  int ju = j0;
  int u = unit_of(ju);
  if (u >= n_units) return;
  int4 d = units[u];
  {
    int SR[C::SPT];
    fetch_rows(d, SR);
    put_rows(SR);
  }
  __syncthreads();

  while (true) {
    const int64_t t0 = d.x;
    const int rows = d.y, cnt = d.w;
    const int ju_n = ju + wpx;
    const int u_n = unit_of(ju_n);
    const bool has_next = u_n < n_units;
    const int4 d_n = has_next ? units[u_n] : make_int4(0, 0, 0, 0);
    // the thread index, made opaque per unit: the LDS addresses of the
    // unit's staging stores and of its 7 x 4 (tap, row block) reads derive
    // from it, and computed once before the unit loop they would hold ~60
    // registers throughout
    int tid_u = tid;
    asm volatile("" : "+v"(tid_u));
    const int s32 = tid_u & 31, h = (tid_u >> 5) & 1;

    // ---- stage the unit's distinct neighbour rows, the zero row and its table ----
    // straight from memory into LDS (global_load_lds: lane l of a wave's load
    // writes the 16 bytes at the load's LDS base + 16 l), every load in
    // flight at once. Slot i of the staging space holds chunk (i % RC) ^
    // swz(s) of staged row s = i / RC; slots past the unit's staged rows
    // load row 0's chunk and are never read.
    if constexpr (NRES < 7) {
      load_a(tap(NRES), 0, AT[0]);
      if constexpr (NRES + 1 < 7) load_a(tap(NRES + 1), 0, AT[1]);
    }
#pragma unroll 2
    for (int j = 0; j < C::MAXJ; ++j) {
      const int base = (j * (C::NT / 64) + w) * 64;
      if (base / RC < cnt) {  // whole waves past the staged rows skip
        const int i = base + lane, sr = i / RC;
        const int row = sbuf[sr < cnt ? sr : 0];
        const _Float16* g = feats + static_cast<int64_t>(row) * CIN + ((i % RC) ^ swz<RC>(sr)) * 8;
        __builtin_amdgcn_global_load_lds(g, (lds_void*)(stg + base), 16, 0, 0);
      }
    }
    // table word e: tap e / 64, rows 2 (e % 64) and + 1 of the unit (units
    // start on even rows, the table's stride is even; words past the unit's
    // rows repeat its last word)
    {
      const int pw = (rows + 1) >> 1;
#pragma unroll 2
      for (int j = 0; j < C::IJ; ++j) {
        const int base = (j * (C::NT / 64) + w) * 64;
        if (base < C::IW) {
          const int e = base + lane, k = e >> 6, p = e & 63;
          const uint32_t* g = sidx2 + k * istride2 + (t0 >> 1) + (p < pw ? p : pw - 1);
          __builtin_amdgcn_global_load_lds(g, (lds_void*)(itab + base), 4, 0, 0);
        }
      }
    }
    if (tid_u < RC) stg[kStageCap * RC + tid_u] = half8{};  // the zero row
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- the next unit's staged-row indices, on their way during the multiplies ----
    int SR_n[C::SPT];
    fetch_rows(d_n, SR_n);

    // ---- this wave's taps over the unit's row blocks; the four waves'
    // partial sums of block rb meet in wave rb, which writes its outputs ----
    auto body = [&](auto nrbc) {
      constexpr int NRB = decltype(nrbc)::value;
      const uint16_t* it16 = reinterpret_cast<const uint16_t*>(itab);
      {
        constexpr int cb = 0;  // the one 32-column block
        float16v acc[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) acc[rb] = float16v{};
        // the staged row of this lane's row in each block at tap k (the zero
        // row when it has none, or past the unit's rows)
        auto load_e = [&](int k, int (&E)[NRB]) {
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) {
            const int r = 32 * rb + s32;
            const int e = r < rows ? it16[k * kStageUnitRows + r] : kStageNone;
            E[rb] = e == kStageNone ? kStageCap : e;
          }
        };
        // one tap, two row blocks at a time: both blocks' operands requested
        // first (and the next tap's staged rows behind the first pair), then
        // the MFMAs alternating between the two blocks' accumulators
        auto multiply = [&](const half8 (&Aw)[KS], const int (&E)[NRB], int k_next, int (&En)[NRB]) {
#pragma unroll
          for (int rp = 0; rp < NRB; rp += 2) {
            const int nb = rp + 1 < NRB ? 2 : 1;
            half8 B[2][KS];
#pragma unroll
            for (int q = 0; q < 2; ++q)
              if (q < nb) {
                const int sw = swz<RC>(E[rp + q]);
#pragma unroll
                for (int st = 0; st < KS; ++st)
                  B[q][st] = stg[E[rp + q] * RC + ((h * KS + st) ^ sw)];
              }
            if (rp == 0) load_e(k_next, En);
#pragma unroll
            for (int st = 0; st < KS; ++st)
#pragma unroll
              for (int q = 0; q < 2; ++q)
                if (q < nb) {
                  if constexpr (IS_BF16)
                    acc[rp + q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, Aw[st]), __builtin_bit_cast(bf16x8, B[q][st]),
                        acc[rp + q], 0, 0, 0);
                  else
                    acc[rp + q] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Aw[st], B[q][st],
                                                                         acc[rp + q], 0, 0, 0);
                }
          }
        };
        int E[2][NRB];
        load_e(tap(0), E[0]);
#pragma unroll
        for (int i = 0; i < 7; ++i) {
          if (i < NRES) {
            if (i < ntaps) multiply(AR[i < NRES ? i : 0], E[i % 2], tap(i + 1), E[(i + 1) % 2]);
          } else {
            if (i < ntaps) multiply(AT[(i - NRES) % 2], E[i % 2], tap(i + 1), E[(i + 1) % 2]);
            if (i + 2 < 7) load_a(tap(i + 2), cb, AT[(i - NRES) % 2]);
          }
        }
        __syncthreads();  // every wave is done with the staged rows and sbuf
        put_rows(SR_n);   // read by the next unit's staging, after the barriers below

        // ---- partial sums of the four waves, in wave order, then the epilogue ----
        constexpr int RPR = C::RPR;
        float4v* red = reinterpret_cast<float4v*>(stg);
#pragma unroll
        for (int rr = 0; rr < NRB; rr += RPR) {
#pragma unroll
          for (int rb = rr; rb < rr + RPR && rb < NRB; ++rb)
            if (w != rb) {
              const int slot = w < rb ? w : w - 1;
#pragma unroll
              for (int a = 0; a < 4; ++a) {
                const float16v& v = acc[rb];
                red[((((rb - rr) * 3 + slot) * 4 + a) * 64) + lane] =
                    float4v{v[4 * a], v[4 * a + 1], v[4 * a + 2], v[4 * a + 3]};
              }
            }
          __syncthreads();
#pragma unroll
          for (int rb = rr; rb < rr + RPR && rb < NRB; ++rb)
            if (w == rb) {
              const int r = 32 * rb + s32;
              const bool live = r < rows;
              const int64_t orow = live ? (order ? order[t0 + r] : t0 + r) : 0;
#pragma unroll
              for (int a = 0; a < 4; ++a) {
                const float16v& v = acc[rb];
                const float4v own = float4v{v[4 * a], v[4 * a + 1], v[4 * a + 2], v[4 * a + 3]};
                // partial sums in wave order: ((p0 + p1) + p2) + p3
                float4v t = rb == 0 ? own : red[(((rb - rr) * 3 + 0) * 4 + a) * 64 + lane];
#pragma unroll
                for (int ww = 1; ww < 4; ++ww) {
                  const int slot = ww < rb ? ww : ww - 1;
                  t += ww == rb ? own : red[(((rb - rr) * 3 + slot) * 4 + a) * 64 + lane];
                }
                if (live) {
                  const int col = 32 * cb + 8 * a + 4 * h;
                  float4v b4 = {0.f, 0.f, 0.f, 0.f};
                  if (bias) b4 = *reinterpret_cast<const float4v*>(bias + col);
                  typedef _Float16 half4 __attribute__((ext_vector_type(4)));
                  const half4 o = {round16<IS_BF16>(t[0] + b4[0]), round16<IS_BF16>(t[1] + b4[1]),
                                   round16<IS_BF16>(t[2] + b4[2]), round16<IS_BF16>(t[3] + b4[3])};
                  // (an ordinary store: the L2 merges a row's 8-byte pieces into whole
                  // lines, where non-temporal stores reached memory as partial lines,
                  // 2.9x the output's bytes)
                  *reinterpret_cast<half4*>(out + orow * COUT + col) = o;
                }
              }
            }
          __syncthreads();  // the partial sums' space (and then stg, itab, sbuf) is free again
        }
      }
    };
    switch ((rows + 31) / 32) {
      case 1: body(std::integral_constant<int, 1>{}); break;
      case 2: body(std::integral_constant<int, 2>{}); break;
      case 3: body(std::integral_constant<int, 3>{}); break;
      default: body(std::integral_constant<int, 4>{}); break;
    }
    if (!has_next) break;
    ju = ju_n;
    d = d_n;
  }
}

// 32 -> 64 channels (the input gradient of a 64 -> 32 layer): both 32-column
// blocks accumulate in one pass over the staged rows, so each staged-row
// fragment read feeds two MFMAs and every tap's weights of both blocks are
// loaded once per unit; the four waves' partial sums meet in the staging
// space one row block (both column blocks) at a time, added in wave order as
// in k_fwd_staged (the same sums, the same bits).
template <bool IS_BF16>
__global__ __launch_bounds__(256, 2) void k_fwd_staged_c64(
    const int4* __restrict__ units, int n_units, int per_xcd, int wpx,
    const int32_t* __restrict__ srows, const uint32_t* __restrict__ sidx2, int64_t istride2,
    const int32_t* __restrict__ order, int64_t n, const _Float16* __restrict__ feats,
    const _Float16* __restrict__ wp, const float* __restrict__ bias, _Float16* __restrict__ out) {
  constexpr int CIN = 32, COUT = 64;
  using C = CfgSt<CIN, COUT>;
  constexpr int KS = C::KS, RC = C::RC, NCB = C::NCB;
  static_assert(NCB == 2 && 2 * C::RED <= C::STG * 1, "a row block's partial sums fit the staging space");
  __shared__ half8 stg[C::STG];
  __shared__ uint32_t itab[C::IW];      // [27][128] staged rows of the unit's rows, two per word
  __shared__ int32_t sbuf[kStageCap];   // the unit's staged rows (caller rows)

  const int bid = blockIdx.x;
  const int xcd = bid & 7, j0 = bid >> 3;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ntaps = (kTaps3 - w + 3) / 4;  // this wave's taps k = w + 4 i
  // taps past the wave's last load tap 26 again and go unused, so that no
  // load sits in a branch (the compiler's waits for loads would otherwise
  // assume the fewest in flight after the branch)
  auto tap = [&](int i) { return w + 4 * i < kTaps3 ? w + 4 * i : kTaps3 - 1; };

  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wp, static_cast<uint32_t>(kTaps3 * CIN * COUT * 2));
  // the weights of tap k, both column blocks (1 KiB per K step, in fragment order)
  auto load_a = [&](int k, half8 (&A)[NCB][KS]) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const uint32_t base = static_cast<uint32_t>(((k * NCB + cb) * KS) * 1024 + lane * 16);
#pragma unroll
      for (int st = 0; st < KS; ++st) A[cb][st] = bload_h8(rw, base + st * 1024);
    }
  };
  // v_mfma_f32_32x32x16: A = weights (lane: column lane%32, K steps st of
  // lane half h = lane/32: channels h CIN/2 + 8 st + 0..7), B = staged rows
  // (lane: row lane%32 of the block, the same channels); D: lane holds row
  // lane%32 and columns 8 a + 4 h + b in register 4 a + b.
  // AT: a two-slot ring of taps' weights, loaded two taps ahead
  half8 AT[2][NCB][KS];

  // a unit's descriptor, staged-row indices (to sbuf) and table words (to
  // itab): requested by fetch_*, stored by put_*
  auto unit_of = [&](int ju) { return ju < per_xcd ? xcd * per_xcd + ju : n_units; };
  auto fetch_rows = [&](const int4& d, int (&SR)[C::SPT]) {
#pragma unroll
    for (int q = 0; q < C::SPT; ++q) {
      const int sr = tid + C::NT * q;
      SR[q] = sr < d.w ? srows[d.z + sr] : -1;
    }
  };
  auto put_rows = [&](const int (&SR)[C::SPT]) {
#pragma unroll
    for (int q = 0; q < C::SPT; ++q) sbuf[tid + C::NT * q] = SR[q];
  };

  int ju = j0;
  int u = unit_of(ju);
  if (u >= n_units) return;
  int4 d = units[u];
  {
    int SR[C::SPT];
    fetch_rows(d, SR);
    put_rows(SR);
  }
  __syncthreads();

  while (true) {
    const int64_t t0 = d.x;
    const int rows = d.y, cnt = d.w;
    const int ju_n = ju + wpx;
    const int u_n = unit_of(ju_n);
    const bool has_next = u_n < n_units;
    const int4 d_n = has_next ? units[u_n] : make_int4(0, 0, 0, 0);
    // the thread index, made opaque per unit: the LDS addresses of the
    // unit's staging stores and of its 7 x 4 (tap, row block) reads derive
    // from it, and computed once before the unit loop they would hold ~60
    // registers throughout
    int tid_u = tid;
    asm volatile("" : "+v"(tid_u));
    const int s32 = tid_u & 31, h = (tid_u >> 5) & 1;

    // ---- stage the unit's distinct neighbour rows, the zero row and its table ----
    // straight from memory into LDS (global_load_lds: lane l of a wave's load
    // writes the 16 bytes at the load's LDS base + 16 l), every load in
    // flight at once. Slot i of the staging space holds chunk (i % RC) ^
    // swz(s) of staged row s = i / RC; slots past the unit's staged rows
    // load row 0's chunk and are never read.
    load_a(tap(0), AT[0]);
    load_a(tap(1), AT[1]);
#pragma unroll 2
    for (int j = 0; j < C::MAXJ; ++j) {
      const int base = (j * (C::NT / 64) + w) * 64;
      if (base / RC < cnt) {  // whole waves past the staged rows skip
        const int i = base + lane, sr = i / RC;
        const int row = sbuf[sr < cnt ? sr : 0];
        const _Float16* g = feats + static_cast<int64_t>(row) * CIN + ((i % RC) ^ swz<RC>(sr)) * 8;
        __builtin_amdgcn_global_load_lds(g, (lds_void*)(stg + base), 16, 0, 0);
      }
    }
    // table word e: tap e / 64, rows 2 (e % 64) and + 1 of the unit (units
    // start on even rows, the table's stride is even; words past the unit's
    // rows repeat its last word)
    {
      const int pw = (rows + 1) >> 1;
#pragma unroll 2
      for (int j = 0; j < C::IJ; ++j) {
        const int base = (j * (C::NT / 64) + w) * 64;
        if (base < C::IW) {
          const int e = base + lane, k = e >> 6, p = e & 63;
          const uint32_t* g = sidx2 + k * istride2 + (t0 >> 1) + (p < pw ? p : pw - 1);
          __builtin_amdgcn_global_load_lds(g, (lds_void*)(itab + base), 4, 0, 0);
        }
      }
    }
    if (tid_u < RC) stg[kStageCap * RC + tid_u] = half8{};  // the zero row
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- the next unit's staged-row indices, on their way during the multiplies ----
    int SR_n[C::SPT];
    fetch_rows(d_n, SR_n);

    // ---- this wave's taps over the unit's row blocks; the four waves'
    // partial sums of block rb meet in wave rb, which writes its outputs ----
    auto body = [&](auto nrbc) {
      constexpr int NRB = decltype(nrbc)::value;
      const uint16_t* it16 = reinterpret_cast<const uint16_t*>(itab);
      float16v acc[NRB][NCB];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = float16v{};
      // the staged row of this lane's row in each block at tap k (the zero
      // row when it has none, or past the unit's rows)
      auto load_e = [&](int k, int (&E)[NRB]) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const int r = 32 * rb + s32;
          const int e = r < rows ? it16[k * kStageUnitRows + r] : kStageNone;
          E[rb] = e == kStageNone ? kStageCap : e;
        }
      };
      // one tap, two row blocks at a time: both blocks' operands requested
      // first (and the next tap's staged rows behind the first pair), then
      // the MFMAs of both column blocks, alternating over four accumulators
      auto multiply = [&](const half8 (&Aw)[NCB][KS], const int (&E)[NRB], int k_next,
                          int (&En)[NRB]) {
#pragma unroll
        for (int rp = 0; rp < NRB; rp += 2) {
          const int nb = rp + 1 < NRB ? 2 : 1;
          half8 B[2][KS];
#pragma unroll
          for (int q = 0; q < 2; ++q)
            if (q < nb) {
              const int sw = swz<RC>(E[rp + q]);
#pragma unroll
              for (int st = 0; st < KS; ++st) B[q][st] = stg[E[rp + q] * RC + ((h * KS + st) ^ sw)];
            }
          if (rp == 0) load_e(k_next, En);
#pragma unroll
          for (int st = 0; st < KS; ++st)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
              for (int cb = 0; cb < NCB; ++cb)
                if (q < nb) {
                  if constexpr (IS_BF16)
                    acc[rp + q][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, Aw[cb][st]), __builtin_bit_cast(bf16x8, B[q][st]),
                        acc[rp + q][cb], 0, 0, 0);
                  else
                    acc[rp + q][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Aw[cb][st], B[q][st],
                                                                             acc[rp + q][cb], 0, 0, 0);
                }
        }
      };
      int E[2][NRB];
      load_e(tap(0), E[0]);
#pragma unroll
      for (int i = 0; i < 7; ++i) {
        if (i < ntaps) multiply(AT[i % 2], E[i % 2], tap(i + 1), E[(i + 1) % 2]);
        if (i + 2 < 7) load_a(tap(i + 2), AT[i % 2]);
      }
      __syncthreads();  // every wave is done with the staged rows and sbuf
      put_rows(SR_n);   // read by the next unit's staging, after the barriers below

      // ---- partial sums of the four waves, one row block (both column
      // blocks) at a time, in wave order, then the epilogue ----
      float4v* red = reinterpret_cast<float4v*>(stg);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        if (w != rb) {
          const int slot = w < rb ? w : w - 1;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
              const float16v& v = acc[rb][cb];
              red[(((cb * 3 + slot) * 4 + a) * 64) + lane] =
                  float4v{v[4 * a], v[4 * a + 1], v[4 * a + 2], v[4 * a + 3]};
            }
        }
        __syncthreads();
        if (w == rb) {
          const int r = 32 * rb + s32;
          const bool live = r < rows;
          const int64_t orow = live ? (order ? order[t0 + r] : t0 + r) : 0;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
              const float16v& v = acc[rb][cb];
              const float4v own = float4v{v[4 * a], v[4 * a + 1], v[4 * a + 2], v[4 * a + 3]};
              // partial sums in wave order: ((p0 + p1) + p2) + p3
              float4v t = rb == 0 ? own : red[((cb * 3 + 0) * 4 + a) * 64 + lane];
#pragma unroll
              for (int ww = 1; ww < 4; ++ww) {
                const int slot = ww < rb ? ww : ww - 1;
                t += ww == rb ? own : red[((cb * 3 + slot) * 4 + a) * 64 + lane];
              }
              if (live) {
                const int col = 32 * cb + 8 * a + 4 * h;
                float4v b4 = {0.f, 0.f, 0.f, 0.f};
                if (bias) b4 = *reinterpret_cast<const float4v*>(bias + col);
                typedef _Float16 half4 __attribute__((ext_vector_type(4)));
                const half4 o = {round16<IS_BF16>(t[0] + b4[0]), round16<IS_BF16>(t[1] + b4[1]),
                                 round16<IS_BF16>(t[2] + b4[2]), round16<IS_BF16>(t[3] + b4[3])};
                *reinterpret_cast<half4*>(out + orow * COUT + col) = o;
              }
            }
        }
        __syncthreads();  // the partial sums' space (and then stg, itab, sbuf) is free again
      }
    };
    switch ((rows + 31) / 32) {
      case 1: body(std::integral_constant<int, 1>{}); break;
      case 2: body(std::integral_constant<int, 2>{}); break;
      case 3: body(std::integral_constant<int, 3>{}); break;
      default: body(std::integral_constant<int, 4>{}); break;
    }
    if (!has_next) break;
    ju = ju_n;
    d = d_n;
  }
}

// workgroups of one instance that a CU holds at once (cached)

template <bool IS_BF16>
int launch_staged_c64(const Map& m, const _Float16* feats, const _Float16* wp, const float* bias,
                      _Float16* out, hipStream_t stream) {
  static const int per_cu = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &nb, reinterpret_cast<const void*>(k_fwd_staged_c64<IS_BF16>), CfgSt<32, 64>::NT, 0) !=
        hipSuccess)
      nb = 1;
    return nb < 1 ? 1 : nb;
  }();
  const Staged& S = m.staged;
  if (S.n_units > (int64_t{1} << 28))
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "too many staged units");
  int dev = 0, cus = 256;
  SUBMCONV_HIP_CHECK(hipGetDevice(&dev));
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int per_xcd = static_cast<int>((S.n_units + 7) / 8);
  const int slots = (cus < 8 ? 1 : cus / 8) * per_cu;
  const int wpx = per_xcd < slots ? per_xcd : slots;
  k_fwd_staged_c64<IS_BF16><<<static_cast<unsigned>(8 * wpx), CfgSt<32, 64>::NT, 0, stream>>>(
      S.units, static_cast<int>(S.n_units), per_xcd, wpx, S.rows,
      reinterpret_cast<const uint32_t*>(S.idx), staged_idx_stride(m.n) / 2, m.order, m.n, feats,
      wp, bias, out);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

// workgroups of one instance that a CU holds at once (cached)
template <int CIN, int COUT, bool IS_BF16>
int staged_per_cu() {
  static const int per_cu = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &nb, reinterpret_cast<const void*>(k_fwd_staged<CIN, COUT, IS_BF16>),
            CfgSt<CIN, COUT>::NT, 0) != hipSuccess)
      nb = 1;
    return nb < 1 ? 1 : nb;
  }();
  return per_cu;
}

template <int CIN, int COUT, bool IS_BF16>
int launch_staged(const Map& m, const _Float16* feats, const _Float16* wp, const float* bias,
                  _Float16* out, hipStream_t stream) {
  const Staged& S = m.staged;
  if (S.n_units > (int64_t{1} << 28))
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "too many staged units");
  int dev = 0, cus = 256;
  SUBMCONV_HIP_CHECK(hipGetDevice(&dev));
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int per_xcd = static_cast<int>((S.n_units + 7) / 8);
  // as many workgroups as the CUs hold at once, dealt evenly to the 8 XCDs
  const int slots = (cus < 8 ? 1 : cus / 8) * staged_per_cu<CIN, COUT, IS_BF16>();
  const int wpx = per_xcd < slots ? per_xcd : slots;
  k_fwd_staged<CIN, COUT, IS_BF16><<<static_cast<unsigned>(8 * wpx), CfgSt<CIN, COUT>::NT, 0,
                                     stream>>>(S.units, static_cast<int>(S.n_units), per_xcd, wpx,
                                               S.rows, reinterpret_cast<const uint32_t*>(S.idx),
                                               staged_idx_stride(m.n) / 2, m.order, m.n, feats, wp,
                                               bias, out);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

template <bool IS_BF16>
int staged_typed(const Map& m, int cin, int cout, const _Float16* feats, const _Float16* wp,
                 const float* bias, _Float16* out, hipStream_t stream) {
  if (cout == 256) return forward_staged_wide(m, cin, IS_BF16, feats, wp, bias, out, stream);
  if (cin == 64) return launch_staged<64, 32, IS_BF16>(m, feats, wp, bias, out, stream);
  if (cout == 64) return launch_staged_c64<IS_BF16>(m, feats, wp, bias, out, stream);
  return launch_staged<32, 32, IS_BF16>(m, feats, wp, bias, out, stream);
}

}  // namespace

int staged_count(const int32_t* nbr, int64_t n, const StagedTemps& tp, hipStream_t stream) {
  if (tp.n_tiles <= 0) return SUBMCONV_OK;
  if (tp.n_tiles > INT32_MAX) return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "too many tiles");
  k_stage_count<<<static_cast<unsigned>(tp.n_tiles), kPlanThreads, 0, stream>>>(
      nbr, n, tp.tile_units, tp.tile_nu, tp.tile_ns);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  k_stage_scan<<<1, 1024, 0, stream>>>(tp.tile_nu, tp.tile_ns, tp.n_tiles, tp.unit_off,
                                       tp.staged_off, tp.totals);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

int staged_fill(const int32_t* nbr, int64_t n, const StagedTemps& tp, const Staged& plan,
                hipStream_t stream) {
  if (tp.n_tiles <= 0) return SUBMCONV_OK;
  k_stage_fill<<<static_cast<unsigned>(tp.n_tiles), kPlanThreads, 0, stream>>>(
      nbr, n, tp.tile_units, tp.tile_nu, tp.unit_off, tp.staged_off, plan.units, plan.rows,
      plan.idx, staged_idx_stride(n));
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

bool staged_shape(int cin, int cout) {
  // (64 -> 64 needs more registers than two waves per SIMD have)
  return (cin == 32 && (cout == 32 || cout == 64)) || (cin == 64 && cout == 32) ||
         ((cin == 128 || cin == 256) && cout == 256);
}

bool staged_takes(const Map& m, int ksize, int cin, int cout) {
  return ksize == 3 && m.staged.n_units > 0 && staged_shape(cin, cout);
}

int forward_staged(const Map& m, int cin, int cout, bool bf16, const _Float16* feats,
                   const _Float16* wp, const float* bias, _Float16* out, hipStream_t stream) {
  if (bf16) return staged_typed<true>(m, cin, cout, feats, wp, bias, out, stream);
  return staged_typed<false>(m, cin, cout, feats, wp, bias, out, stream);
}

}  // namespace submconv
