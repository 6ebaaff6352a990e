// SubMConv3d weight gradient on gfx950.
//
// dW[k] = sum over the pairs (i, j) of tap k, j the row at c_i + d_k, of the
// outer product feats[j]^T grad_out[i]: the gradient of the forward's
// per-tap products feats[j] @ W[k] (the issue #1 thread lists a
// weight-gradient kernel next to the forward; this is its sum).
//
// The pairs of a tap are the map's per-tile lists {j, row in tile}. A
// workgroup takes one tap and a run of consecutive tiles; for each group of
// 32 pairs it gathers the 32 feature rows and the 32 output-gradient rows,
// stores both channel-major in LDS (so that the 32 pairs become the MFMA's
// K dimension), and accumulates v_mfma_f32_32x32x16_f16 products: wave w owns
// output columns 32w..32w+31 and every block of 32 input channels. Each
// workgroup writes its fp32 partial dW[k] to a workspace; a second kernel
// adds the partials of a tap in a fixed order, so the result does not depend
// on scheduling.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <tuple>
#include <climits>
#include <mutex>
#include <type_traits>
#include <utility>

#include "submconv_internal.h"

// Workspace of submconv_backward_weight_noalloc, for callers that cannot
// allocate: device memory of the library's code object, one copy per device
// from the time the library's kernels load on it until the process ends. In
// host code the array's name is a stand-in, not a device address: host code
// uses only the address hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocScratchBytes = size_t{32} << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace submconv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kPairs = 32;          // pairs per group
constexpr int kRowPad = kPairs + 8; // LDS row (one channel): 32 pairs + 8 halves of padding
constexpr int kTargetBlocks = 1024; // workgroups to aim for (taps x tile runs)
constexpr int kBlocksPerCU = 2;     // workgroups per compute unit, pipelined kernel
constexpr double kGroupsSmall = 64;  // groups per workgroup, pipelined kernel, < 4 waves

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ half8 bload_h8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <int CIN, int COUT>
struct WCfg {
  static constexpr int NW = COUT / 32;   // waves, one per 32 output columns
  static constexpr int NT = 64 * NW;
  static constexpr int MB = CIN / 32;    // 32-channel blocks of the input
  static constexpr int FC = CIN / 8;     // 16-byte chunks of a feature row
  static constexpr int YC = COUT / 8;    // 16-byte chunks of a gradient row
  static constexpr int FI = (kPairs * FC + NT - 1) / NT;  // feature chunks per thread
  static constexpr int YI = (kPairs * YC + NT - 1) / NT;  // gradient chunks per thread
  static_assert(CIN % 32 == 0 && COUT % 32 == 0 && CIN <= 256 && COUT <= 256, "channels");
};

// grid: blockIdx.x = run * K + tap index; tiles [run * tpr, (run+1) * tpr).
template <int CIN, int COUT>
__global__ __launch_bounds__(2 * COUT) void k_bwd_weight(
    const int2* __restrict__ ent, const int32_t* __restrict__ tile_off,
    const uint16_t* __restrict__ tile_cnt, const int32_t* __restrict__ order, int64_t n,
    int32_t n_tiles, int32_t tile_rows, int32_t K, int32_t tpr, const _Float16* __restrict__ feats,
    const _Float16* __restrict__ grad_out, float* __restrict__ partial, int32_t n_pairs) {
  using C = WCfg<CIN, COUT>;
  static_assert(C::NT == 2 * COUT, "launch bounds");
  __shared__ _Float16 ft[CIN * kRowPad];   // feature rows, channel-major
  __shared__ _Float16 yt[COUT * kRowPad];  // gradient rows, channel-major

  const int kp = blockIdx.x % K;           // processing position (tap) of this block
  const int run = blockIdx.x / K;
  const int p = K == kTaps3 ? kp : 0;      // position in the per-tile lists
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int t_begin = run * tpr;
  const int t_end = min(t_begin + tpr, n_tiles);

  const __amdgpu_buffer_rsrc_t rf = make_rsrc(feats, static_cast<uint32_t>(n * CIN * 2));
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(grad_out, static_cast<uint32_t>(n * COUT * 2));

  float16v acc[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) acc[mb] = float16v{};

  // A operand (lane: channel 32*mb + lane%32, pairs 16*kk + 8*(lane/32) + 0..7)
  // and B operand (lane: column 32*w + lane%32, same pairs), from LDS.
  const int s32 = lane & 31;
  const int h = lane >> 5;

  for (int t = t_begin; t < t_end; ++t) {
    // entries of position p in tile t
    int before = 0;
    for (int q = 0; q < p; ++q) before += tile_cnt[static_cast<int64_t>(t) * kTaps3 + q];
    const int cnt = tile_cnt[static_cast<int64_t>(t) * kTaps3 + p];  // p = 0: every row of the tile
    const int64_t first = static_cast<int64_t>(tile_off[t]) + before;
    for (int g0 = 0; g0 < cnt; g0 += kPairs) {
      // gather 32 pairs into registers
      half8 fv[C::FI], yv[C::YI];
      int fpair[C::FI], fch[C::FI], ypair[C::YI], ych[C::YI];
#pragma unroll
      for (int i = 0; i < C::FI; ++i) {
        const int c = tid + C::NT * i;
        fpair[i] = c % kPairs;
        fch[i] = c / kPairs;
        uint32_t off = kOob;
        if (fch[i] < C::FC && g0 + fpair[i] < cnt) {
          const int2 e = ent[first + g0 + fpair[i]];
          off = static_cast<uint32_t>(e.x) * (CIN * 2) + fch[i] * 16;
        }
        fv[i] = bload_h8(rf, off);
      }
#pragma unroll
      for (int i = 0; i < C::YI; ++i) {
        const int c = tid + C::NT * i;
        ypair[i] = c % kPairs;
        ych[i] = c / kPairs;
        uint32_t off = kOob;
        if (ych[i] < C::YC && g0 + ypair[i] < cnt) {
          const int2 e = ent[first + g0 + ypair[i]];
          const int64_t t_row = int64_t{t} * tile_rows + e.y;
          const int64_t row = order ? order[t_row] : t_row;
          off = static_cast<uint32_t>(row) * (COUT * 2) + ych[i] * 16;
        }
        yv[i] = bload_h8(rg, off);
      }
      __syncthreads();  // the previous group's fragments have been read
#pragma unroll
      for (int i = 0; i < C::FI; ++i) {
        if (fch[i] < C::FC) {
#pragma unroll
          for (int q = 0; q < 8; ++q) ft[(fch[i] * 8 + q) * kRowPad + fpair[i]] = fv[i][q];
        }
      }
#pragma unroll
      for (int i = 0; i < C::YI; ++i) {
        if (ych[i] < C::YC) {
#pragma unroll
          for (int q = 0; q < 8; ++q) yt[(ych[i] * 8 + q) * kRowPad + ypair[i]] = yv[i][q];
        }
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kPairs / 16; ++kk) {
        const half8 b = *reinterpret_cast<const half8*>(&yt[(32 * w + s32) * kRowPad + 16 * kk + 8 * h]);
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
          const half8 a = *reinterpret_cast<const half8*>(&ft[(32 * mb + s32) * kRowPad + 16 * kk + 8 * h]);
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[mb], 0, 0, 0);
        }
      }
    }
  }
  // D: lane holds column 32w + lane%32 and channels 32mb + 8a + 4h + b in
  // register 4a + b
  float* dst = partial + static_cast<int64_t>(blockIdx.x) * CIN * COUT;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int ci = 32 * mb + 8 * a + 4 * h + b;
        dst[static_cast<int64_t>(ci) * COUT + 32 * w + s32] = acc[mb][4 * a + b];
      }
    }
  }
  (void)n_pairs;
}

// ---------------------------------------------------------------------------
// Pipelined weight-gradient kernel for Cin, Cout in {32, 64, 128, 256}
// ---------------------------------------------------------------------------
//
// Same decomposition and partials as k_bwd_weight, restructured as a software
// pipeline over the groups of 32 pairs of the workgroup's tap. The gathered
// feature and gradient rows go to LDS as they are (16-byte chunks, XOR
// swizzled rows); the MFMA operands, 8 consecutive pairs of one channel, are
// read from those rows with ds_read_b64_tr_b16, which transposes 16 lanes'
// 4-element row pieces into 4-element column pieces. Group g: list entries
// requested in step g-5, gradient rows resolved (through the processing
// order) in step g-3, rows gathered in step g-2, stored to LDS slot g%2 in
// step g-1, multiplied in step g. Wave (wr, wc) owns input-channel blocks
// wr*RB.. and output-column blocks wc*CB.. of dW[k] in registers.

typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int2 bload_i2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(int2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ int bload_i1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

__device__ __forceinline__ int excl_scan_wave(int v, int lane) {
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x - v;
}

// register tile of a wave: RB x CB blocks of 32 x 32 (input x output channels)
constexpr int pp_rb(int cin, int cout) {
  return ((cin / 32) % 4 == 0 && (cin / 32) * (cout / 32) > 16) ? 4 : ((cin / 32) % 2 == 0 ? 2 : 1);
}
constexpr int pp_cb(int cout) { return (cout / 32) % 2 == 0 ? 2 : 1; }
constexpr int pp_waves(int cin, int cout) {
  return (cin / 32 / pp_rb(cin, cout)) * (cout / 32 / pp_cb(cout));
}

template <int CIN, int COUT>
struct PCfg {
  static constexpr int MB = CIN / 32, NB = COUT / 32;
  static constexpr int RB = pp_rb(CIN, COUT);
  static constexpr int CB = pp_cb(COUT);
  static constexpr int WR = MB / RB, WC = NB / CB;
  static constexpr int NW = WR * WC;
  static_assert(NW == pp_waves(CIN, COUT), "wave count");
  static constexpr int NT = 64 * NW;
  static constexpr int FC = CIN / 8, YC = COUT / 8;  // 16-byte chunks per row
  static constexpr int FT = kPairs * FC, YT = kPairs * YC;
  static constexpr int CF = FT >= NT ? FT / NT : 1;  // chunks per thread, one row each
  static constexpr int CY = YT >= NT ? YT / NT : 1;
  static constexpr int NF = FT >= NT ? NT : FT;      // threads that gather
  static constexpr int NY = YT >= NT ? NT : YT;
  static constexpr int TW = 64;                      // tiles per schedule window
  static_assert((CIN == 32 || CIN == 64 || CIN == 128 || CIN == 256) &&
                    (COUT == 32 || COUT == 64 || COUT == 128 || COUT == 256),
                "channels");
  static_assert(FT % NT == 0 || NT % FT == 0, "feature chunk split");
  static_assert(YT % NT == 0 || NT % YT == 0, "gradient chunk split");
  static_assert(FC % CF == 0 && YC % CY == 0, "a thread's chunks share a row");
};

// Work split of the pipelined weight gradient. Blocks [0, runs0) take the
// centre (position 0, every row of a tile) in runs of tpr0 tiles; block
// runs0 + r*26 + (p-1) takes position p >= 1, tiles [r*tpr, (r+1)*tpr). The
// positions of one tile range are neighbours in the grid, so blocks that run
// together gather the same rows and share the L2.
struct WSplit {
  int32_t np;  // positions: 27, or 1 for a 1x1x1 kernel
  int32_t runs0, tpr0, runs, tpr;
  __host__ __device__ int32_t blocks() const { return runs0 + (np - 1) * runs; }
  __host__ __device__ int32_t first(int p) const { return p == 0 ? 0 : runs0 + p - 1; }
  __host__ __device__ int32_t count(int p) const { return p == 0 ? runs0 : runs; }
  __host__ __device__ int32_t stride(int p) const { return p == 0 ? 1 : np - 1; }
};

template <int CIN, int COUT, bool ORD>
__global__ __launch_bounds__((PCfg<CIN, COUT>::NT)) void k_bwd_weight_pp(
    const int2* __restrict__ ent, const int32_t* __restrict__ tile_off,
    const uint16_t* __restrict__ tile_cnt, const int32_t* __restrict__ order, int64_t n,
    int32_t n_tiles, int32_t tile_rows, const WSplit ws, const _Float16* __restrict__ feats,
    const _Float16* __restrict__ grad_out, float* __restrict__ partial, int32_t n_pairs) {
  using C = PCfg<CIN, COUT>;
  constexpr int FC = C::FC, YC = C::YC, CF = C::CF, CY = C::CY, RB = C::RB, CB = C::CB;
  __shared__ half8 fs[2][kPairs * FC];  // feature rows of a group, pair-major
  __shared__ half8 ys[2][kPairs * YC];  // gradient rows of a group

  const int bid = blockIdx.x;
  int p, t_begin;
  if (bid < ws.runs0) {
    p = 0;
    t_begin = bid * ws.tpr0;
  } else {
    const int b = bid - ws.runs0;
    p = 1 + b % (ws.np - 1);
    t_begin = (b / (ws.np - 1)) * ws.tpr;
  }
  const int t_end = min(t_begin + (p == 0 ? ws.tpr0 : ws.tpr), n_tiles);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = w / C::WC, wc = w - (w / C::WC) * C::WC;

  const __amdgpu_buffer_rsrc_t rf = make_rsrc(feats, static_cast<uint32_t>(n * CIN * 2));
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(grad_out, static_cast<uint32_t>(n * COUT * 2));
  const __amdgpu_buffer_rsrc_t re = make_rsrc(ent, static_cast<uint32_t>(n_pairs + 1) * 8u);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(order, ORD ? static_cast<uint32_t>(n * 4) : 0u);
  const uint32_t e_none = static_cast<uint32_t>(n_pairs) * 8u;  // the closing {-1, -1} entry

  // gather roles: CF consecutive chunks of one feature row, CY of one
  // gradient row
  const bool gf = tid < C::NF, gy = tid < C::NY;
  const int pf = (tid * CF) / FC, cf0 = (tid * CF) % FC;
  const int py = (tid * CY) / YC, cy0 = (tid * CY) % YC;

  float16v acc[RB][CB];
#pragma unroll
  for (int a = 0; a < RB; ++a)
#pragma unroll
    for (int b = 0; b < CB; ++b) acc[a][b] = float16v{};

  // transposed operand reads: lane (group gq = lane/16, s = lane%16) names
  // row 8*(gq/2) + 4*r + s/4 and channels 16*(gq%2) + 4*(s%4).. of a 32-row,
  // 32-channel block; it receives channel 16*(gq%2) + s of rows
  // 8*(gq/2) + 4*r + 0..3
  const int gq = lane >> 4, sl = lane & 15;
  auto tr_addr = [&](int rc, int blk, int kk, int r) {  // in halves, rc chunks per row
    const int row = 16 * kk + 8 * (gq >> 1) + 4 * r + (sl >> 2);
    const int ch = 32 * blk + 16 * (gq & 1) + 4 * (sl & 3);
    return row * rc * 8 + (((ch >> 3) ^ (row & (rc - 1))) << 3) + (((ch >> 2) & 1) << 2);
  };
  auto operand = [&](const half8* base, int rc, int blk, int kk) {
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const _Float16* hb = reinterpret_cast<const _Float16*>(base);
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4s*)(hb + tr_addr(rc, blk, kk, 0)));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4s*)(hb + tr_addr(rc, blk, kk, 1)));
    return __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto lds_barrier = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  for (int wb = t_begin; wb < t_end; wb += C::TW) {
    // ---- schedule of this window: lane i holds tile wb + i ----
    const int nt = min(C::TW, t_end - wb);
    int cnt = 0, off = 0;
    if (lane < nt) {
      const int64_t tb = static_cast<int64_t>(wb + lane) * kTaps3;
      int before = 0;
      for (int q = 0; q < p; ++q) before += tile_cnt[tb + q];
      cnt = tile_cnt[tb + p];  // p = 0: every row of the tile
      off = tile_off[wb + lane] + before;
    }
    const int ng = (cnt + kPairs - 1) / kPairs;
    const int gsx = excl_scan_wave(ng, lane);
    const int G = __builtin_amdgcn_readlane(gsx + ng, 63);
    if (G == 0) continue;
    const int s_gs = lane < nt ? gsx : INT_MAX;
    const int s_offg = off - kPairs * gsx;
    const int s_end = off + cnt;
    struct Grp {
      int start, cnt, tile;
    };
    auto grp = [&](int g) -> Grp {
      Grp r{0, 0, wb};
      if (g < 0) return r;  // before the window: nothing
      const uint64_t m = __ballot(s_gs <= g);
      const int i = 63 - __builtin_clzll(m);
      r.start = __builtin_amdgcn_readlane(s_offg, i) + kPairs * g;
      const int c = __builtin_amdgcn_readlane(s_end, i) - r.start;
      r.cnt = c < kPairs ? c : kPairs;  // <= 0 past the window's pairs
      r.tile = wb + i;
      return r;
    };

    // ---- pipeline stages ----
    // group g: list entries requested in step g-8, rows resolved in step
    // g-6 (the gradient row through the processing order), rows gathered in
    // step g-4, stored to LDS slot g%2 in step g-1, multiplied in step g
    struct Ent {
      int2 f, y;
    };
    struct Rows {
      int f, y;   // feature row (-1: none), caller row of the gradient row
      bool ylive;
    };
    struct Chunks {
      half8 f[CF], y[CY];
    };
    auto load_entries = [&](const Grp& g) {
      Ent e;
      e.f = bload_i2(re, gf && pf < g.cnt ? static_cast<uint32_t>(g.start + pf) * 8u : e_none);
      if constexpr (C::NF == C::NY && CF * YC == CY * FC) {
        e.y = e.f;  // the same pair
      } else {
        e.y = bload_i2(re, gy && py < g.cnt ? static_cast<uint32_t>(g.start + py) * 8u : e_none);
      }
      return e;
    };
    auto rows_of = [&](const Ent& e, const Grp& g) {
      Rows r;
      r.f = e.f.x;
      r.ylive = e.y.y >= 0;
      const int t_row = g.tile * tile_rows + e.y.y;
      if constexpr (ORD)
        r.y = bload_i1(ro, r.ylive ? static_cast<uint32_t>(t_row) * 4u : kOob);
      else
        r.y = t_row;
      return r;
    };
    auto load_chunks = [&](const Rows& r, Chunks& d) {
#pragma unroll
      for (int k = 0; k < CF; ++k)
        d.f[k] = bload_h8(rf, r.f >= 0 ? static_cast<uint32_t>(r.f) * (CIN * 2) + (cf0 + k) * 16
                                       : kOob);
#pragma unroll
      for (int k = 0; k < CY; ++k)
        d.y[k] = bload_h8(rg, r.ylive ? static_cast<uint32_t>(r.y) * (COUT * 2) + (cy0 + k) * 16
                                      : kOob);
    };
    auto store_chunks = [&](int slot, const Chunks& d) {
      if (gf) {
#pragma unroll
        for (int k = 0; k < CF; ++k) fs[slot][pf * FC + ((cf0 + k) ^ (pf & (FC - 1)))] = d.f[k];
      }
      if (gy) {
#pragma unroll
        for (int k = 0; k < CY; ++k) ys[slot][py * YC + ((cy0 + k) ^ (py & (YC - 1)))] = d.y[k];
      }
    };
    auto multiply = [&](int slot) {
#pragma unroll
      for (int kk = 0; kk < kPairs / 16; ++kk) {
        half8 bo[CB];
#pragma unroll
        for (int b = 0; b < CB; ++b) bo[b] = operand(ys[slot], YC, wc * CB + b, kk);
#pragma unroll
        for (int a = 0; a < RB; ++a) {
          const half8 ao = operand(fs[slot], FC, wr * RB + a, kk);
#pragma unroll
          for (int b = 0; b < CB; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ao, bo[b], acc[a][b], 0, 0, 0);
        }
      }
    };

    // the rings start empty (masked entries, no rows); steps -8..-1 fill them
    Ent E[4];
    Rows RW[4];
    Chunks D[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      E[k].f = E[k].y = int2{-1, -1};
      RW[k] = Rows{-1, 0, false};
#pragma unroll
      for (int q = 0; q < CF; ++q) D[k].f[q] = half8{};
#pragma unroll
      for (int q = 0; q < CY; ++q) D[k].y[q] = half8{};
    }
    auto step = [&](int g, auto ic) {
      constexpr int i = decltype(ic)::value;                 // g mod 4
      store_chunks((i + 1) & 1, D[(i + 1) & 3]);             // group g+1
      if (g >= 0 && g < G) multiply(i & 1);                  // group g, stored last step
      load_chunks(RW[i], D[i]);                              // group g+4
      RW[(i + 2) & 3] = rows_of(E[(i + 2) & 3], grp(g + 6)); // group g+6
      E[i] = load_entries(grp(g + 8));                       // group g+8
      lds_barrier();
    };
    for (int g0 = -8; g0 < G; g0 += 4) {
      step(g0, std::integral_constant<int, 0>{});
      step(g0 + 1, std::integral_constant<int, 1>{});
      step(g0 + 2, std::integral_constant<int, 2>{});
      step(g0 + 3, std::integral_constant<int, 3>{});
    }
  }

  // D: lane holds column 32*cb + lane%32 and channels 32*rb + 8a + 4h + b in
  // register 4a + b
  const int h = lane >> 5, s32 = lane & 31;
  float* dst = partial + static_cast<int64_t>(bid) * CIN * COUT;
#pragma unroll
  for (int a = 0; a < RB; ++a)
#pragma unroll
    for (int b = 0; b < CB; ++b)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          const int ci = 32 * (wr * RB + a) + 8 * a4 + 4 * h + b4;
          const int co = 32 * (wc * CB + b) + s32;
          dst[static_cast<int64_t>(ci) * COUT + co] = acc[a][b][4 * a4 + b4];
        }
}

// dW[tap_at(kp)] = the sum of the partials of position kp's blocks. A
// workgroup takes 64 float4s of one position; thread (s, c) adds the
// position's runs s, s+kRedStrands, ... for float4 c in order, then thread
// (0, c) adds the strands' sums in order: a fixed order, so the result does
// not depend on scheduling. (The centre has a run per few tiles, over a
// hundred at 128^3: its strands are the reduction's long pole.)
constexpr int kRedStrands = 16;
__global__ __launch_bounds__(64 * kRedStrands) void k_bwd_weight_reduce_pp(
    const float* __restrict__ partial, const WSplit ws, int cin, int cout, float* __restrict__ dw) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  __shared__ f4 part[kRedStrands][64];
  const int64_t per4 = static_cast<int64_t>(cin) * cout / 4;
  const int64_t chunks = (per4 + 63) / 64;
  const int kp = static_cast<int>(blockIdx.x / chunks);
  const int64_t c4 = (blockIdx.x % chunks) * 64 + (threadIdx.x & 63);
  const int s = threadIdx.x >> 6;
  const f4* p4 = reinterpret_cast<const f4*>(partial);
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  if (c4 < per4) {
    const int n = ws.count(kp), first = ws.first(kp), stride = ws.stride(kp);
    for (int r = s; r < n; r += kRedStrands)
      acc += p4[static_cast<int64_t>(first + r * stride) * per4 + c4];
  }
  part[s][threadIdx.x & 63] = acc;
  __syncthreads();
  if (s == 0 && c4 < per4) {
    f4 t = part[0][threadIdx.x];
#pragma unroll
    for (int q = 1; q < kRedStrands; ++q) t += part[q][threadIdx.x];
    const int k = ws.np == kTaps3 ? tap_at(kp) : 0;
    reinterpret_cast<f4*>(dw)[k * per4 + c4] = t;
  }
}

// dW[tap_at(kp)][ci][co] = sum over runs of partial[run][kp][ci][co], runs in order.
__global__ void k_bwd_weight_reduce(const float* __restrict__ partial, int runs, int K, int cin,
                                    int cout, float* __restrict__ dw) {
  const int64_t per = static_cast<int64_t>(cin) * cout;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= per * K) return;
  const int kp = static_cast<int>(idx / per);
  const int64_t e = idx - kp * per;
  float s = 0.f;
  for (int r = 0; r < runs; ++r) s += partial[(static_cast<int64_t>(r) * K + kp) * per + e];
  const int k = K == kTaps3 ? tap_at(kp) : 0;
  dw[k * per + e] = s;
}

// Plain fallback for channel counts off the MFMA tiling: one thread per
// (tap, ci, co-group of 8) walks the tap's pairs. Deterministic, slow.
__global__ void k_bwd_weight_valu(const int32_t* __restrict__ nbr, const int32_t* __restrict__ order,
                                  int64_t n, int K, const _Float16* __restrict__ feats,
                                  const _Float16* __restrict__ grad_out, int cin, int cout,
                                  float* __restrict__ dw) {
  const int c8n = cout / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(K) * cin * c8n) return;
  const int o8 = static_cast<int>(idx % c8n);
  const int ci = static_cast<int>((idx / c8n) % cin);
  const int k = static_cast<int>(idx / (static_cast<int64_t>(c8n) * cin));
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int64_t t = 0; t < n; ++t) {
    int64_t j;
    if (K == kTaps3) {
      j = nbr[static_cast<int64_t>(k) * n + t];
      if (j < 0) continue;
    } else {
      j = order ? order[t] : t;
    }
    const int64_t i = order ? order[t] : t;
    const float f = static_cast<float>(feats[j * cin + ci]);
    const half8 g = *reinterpret_cast<const half8*>(grad_out + i * cout + o8 * 8);
#pragma unroll
    for (int q = 0; q < 8; ++q) s[q] += f * static_cast<float>(g[q]);
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) dw[(static_cast<int64_t>(k) * cin + ci) * cout + o8 * 8 + q] = s[q];
}

// grad_b[c] = sum over rows of grad_out[row][c]: one workgroup per 8
// columns, each thread a fixed stride of rows, then a fixed-order tree in LDS.
__global__ __launch_bounds__(256) void k_bwd_bias(const _Float16* __restrict__ grad_out, int64_t n,
                                                  int cout, float* __restrict__ grad_b) {
  __shared__ float part[8][257];
  const int c8 = blockIdx.x;
  const int tid = threadIdx.x;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int64_t r = tid; r < n; r += 256) {
    const half8 v = *reinterpret_cast<const half8*>(grad_out + r * cout + c8 * 8);
#pragma unroll
    for (int q = 0; q < 8; ++q) s[q] += static_cast<float>(v[q]);
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) part[q][tid] = s[q];
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) {
#pragma unroll
      for (int q = 0; q < 8; ++q) part[q][tid] += part[q][tid + w];
    }
    __syncthreads();
  }
  if (tid < 8) grad_b[c8 * 8 + tid] = part[tid][0];
}

bool use_mfma_w(int cin, int cout) {
  return cin % 32 == 0 && cout % 32 == 0 && cin <= 256 && cout <= 256;
}

bool use_pp_w(int cin, int cout) {
  auto ok = [](int c) { return c == 32 || c == 64 || c == 128 || c == 256; };
  return ok(cin) && ok(cout);
}

struct Runs {
  int runs, tpr;
};
// the old kernel: every position in the same runs of tpr tiles (at most
// max_blocks workgroups in all)
Runs runs_for(const Map& m, int K, int64_t max_blocks = INT64_MAX) {
  const int64_t nt = m.tiles.n;
  int64_t runs = (kTargetBlocks + K - 1) / K;
  if (runs > max_blocks / K) runs = max_blocks / K;
  if (runs > nt) runs = nt;
  if (runs < 1) runs = 1;
  const int64_t tpr = (nt + runs - 1) / runs;
  runs = (nt + tpr - 1) / tpr;
  return {static_cast<int>(runs), static_cast<int>(tpr)};
}

// compute units of a device, cached
int device_cus(int dev) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  if (dev < 0 || dev >= kMaxDevices) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 256;
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    v = std::max(1, cus);
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// the pipelined kernel: runs from the map's exact group counts (the centre's,
// and the mean of the other positions'). Workgroups of 4 or more waves: at
// most kBlocksPerCU per compute unit, all resident at once (a few blocks
// more than the CUs hold at that count would make some CUs take a third).
// Smaller workgroups: about kGroupsSmall groups each, many per CU.
WSplit split_for(const Map& m, int K, int cin, int cout, int64_t max_blocks = INT64_MAX) {
  WSplit ws{};
  ws.np = K == kTaps3 ? kTaps3 : 1;
  const int64_t nt = m.tiles.n;
  int64_t off = 0;
  for (int p = 1; p < ws.np; ++p) off += m.tiles.pos_groups[p];
  const double g0 = static_cast<double>(m.tiles.pos_groups[0]);
  const double goff = ws.np > 1 ? static_cast<double>(off) / (ws.np - 1) : 0.0;
  auto runs_of = [nt](double groups, double target, int32_t& runs, int32_t& tpr) {
    int64_t r = static_cast<int64_t>(std::ceil(groups / target));
    r = std::max<int64_t>(1, std::min<int64_t>(r, nt));
    const int64_t t = (nt + r - 1) / r;
    tpr = static_cast<int32_t>(t);
    runs = static_cast<int32_t>((nt + t - 1) / t);
  };
  auto fill = [&](double target) {
    runs_of(g0, target, ws.runs0, ws.tpr0);
    if (ws.np > 1) runs_of(goff, target, ws.runs, ws.tpr);
  };
  double target = kGroupsSmall;
  if (pp_waves(cin, cout) >= 4) {
    const int64_t cap = int64_t{device_cus(m.device)} * kBlocksPerCU;
    target = std::max(16.0, (g0 + off) / static_cast<double>(cap));
    fill(target);
    for (int it = 0; it < 200 && ws.blocks() > cap; ++it) {
      target *= 1.02;
      fill(target);
    }
  } else {
    fill(target);
  }
  // longer runs when the partials must fit a fixed workspace (down to one
  // run per position)
  for (int it = 0; it < 400 && ws.blocks() > max_blocks; ++it) {
    target *= 1.05;
    fill(target);
  }
  return ws;
}

template <int CIN, int COUT>
int launch_w(const Map& m, int K, const _Float16* feats, const _Float16* grad_out, float* partial,
             float* dw, int64_t max_blocks, hipStream_t stream) {
  const Tiles& T = m.tiles;
  const int32_t nt = static_cast<int32_t>(T.n), np = static_cast<int32_t>(m.active_pairs);
  if constexpr ((CIN == 32 || CIN == 64 || CIN == 128 || CIN == 256) &&
                (COUT == 32 || COUT == 64 || COUT == 128 || COUT == 256)) {
    constexpr int NT = PCfg<CIN, COUT>::NT;
    const WSplit ws = split_for(m, K, CIN, COUT, max_blocks);
    const unsigned blocks = static_cast<unsigned>(ws.blocks());
    if (m.order)
      k_bwd_weight_pp<CIN, COUT, true><<<blocks, NT, 0, stream>>>(
          T.ent, T.off, T.cnt, m.order, m.n, nt, T.rows, ws, feats, grad_out, partial, np);
    else
      k_bwd_weight_pp<CIN, COUT, false><<<blocks, NT, 0, stream>>>(
          T.ent, T.off, T.cnt, m.order, m.n, nt, T.rows, ws, feats, grad_out, partial, np);
    SUBMCONV_HIP_CHECK(hipGetLastError());
    const int64_t chunks = (int64_t{CIN} * COUT / 4 + 63) / 64;
    k_bwd_weight_reduce_pp<<<static_cast<unsigned>(ws.np * chunks), 64 * kRedStrands, 0, stream>>>(
        partial, ws, CIN, COUT, dw);
  } else {
    const Runs r = runs_for(m, K, max_blocks);
    const int64_t total = static_cast<int64_t>(K) * CIN * COUT;
    k_bwd_weight<CIN, COUT><<<static_cast<unsigned>(r.runs * K), WCfg<CIN, COUT>::NT, 0, stream>>>(
        T.ent, T.off, T.cnt, m.order, m.n, nt, T.rows, K, r.tpr, feats, grad_out, partial, np);
    SUBMCONV_HIP_CHECK(hipGetLastError());
    k_bwd_weight_reduce<<<static_cast<unsigned>((total + 255) / 256), 256, 0, stream>>>(
        partial, r.runs, K, CIN, COUT, dw);
  }
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

template <int CIN>
int dispatch_w(const Map& m, int K, int cout, const _Float16* feats, const _Float16* grad_out,
               float* partial, float* dw, int64_t mb, hipStream_t stream) {
  switch (cout) {
    case 32: return launch_w<CIN, 32>(m, K, feats, grad_out, partial, dw, mb, stream);
    case 64: return launch_w<CIN, 64>(m, K, feats, grad_out, partial, dw, mb, stream);
    case 96: return launch_w<CIN, 96>(m, K, feats, grad_out, partial, dw, mb, stream);
    case 128: return launch_w<CIN, 128>(m, K, feats, grad_out, partial, dw, mb, stream);
    case 160: return launch_w<CIN, 160>(m, K, feats, grad_out, partial, dw, mb, stream);
    case 192: return launch_w<CIN, 192>(m, K, feats, grad_out, partial, dw, mb, stream);
    case 224: return launch_w<CIN, 224>(m, K, feats, grad_out, partial, dw, mb, stream);
    case 256: return launch_w<CIN, 256>(m, K, feats, grad_out, partial, dw, mb, stream);
    default: return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "internal: Cout = %d", cout);
  }
}

// Workspace bytes of the weight gradient's partials with at most max_blocks
// workgroups (0 for the VALU kernel, which needs none).
int64_t workspace_bytes(const Map& m, int cin, int cout, int ksize, int64_t max_blocks) {
  if (!use_mfma_w(cin, cout) || m.n == 0) return 0;
  const int K = ksize == 3 ? kTaps3 : 1;
  // the staged kernel on a dense map, when its partials (all 27 taps per
  // workgroup) fit
  if (const int64_t sb = staged_wgrad_blocks(m, ksize, cin, cout); sb > 0 && sb * K <= max_blocks)
    return sb * K * cin * cout * static_cast<int64_t>(sizeof(float));
  const int64_t blocks = use_pp_w(cin, cout)
                             ? split_for(m, K, cin, cout, max_blocks).blocks()
                             : static_cast<int64_t>(runs_for(m, K, max_blocks).runs) * K;
  return blocks * cin * cout * static_cast<int64_t>(sizeof(float));
}

int check_weight_args(submconv_map_t map, int32_t cin, int32_t cout, int32_t ksize) {
  if (!map) return set_error(SUBMCONV_ERR_INVALID_ARG, "map is NULL");
  if (ksize != 1 && ksize != 3) return set_error(SUBMCONV_ERR_INVALID_ARG, "ksize = %d", ksize);
  if (cin <= 0 || cout <= 0 || cin % 8 || cout % 8 || cin > 1024 || cout > 1024)
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "Cin = %d, Cout = %d", cin, cout);
  return SUBMCONV_OK;
}

// The weight gradient with partials in `workspace` (ws bytes, computed for at
// most max_blocks workgroups).
int backward_weight_impl(const Map& m, const uint16_t* feats, const uint16_t* grad_out,
                                float* grad_w, void* workspace, int64_t ws, int64_t max_blocks,
                                int32_t cin, int32_t cout, int32_t ksize, hipStream_t stream) {
  const int K = ksize == 3 ? kTaps3 : 1;
  if (!grad_w) return set_error(SUBMCONV_ERR_INVALID_ARG, "grad_w is NULL");
  if (m.n == 0) {
    SUBMCONV_HIP_CHECK(hipMemsetAsync(grad_w, 0, sizeof(float) * K * cin * cout, stream));
    return SUBMCONV_OK;
  }
  if (!feats || !grad_out) return set_error(SUBMCONV_ERR_INVALID_ARG, "feats or grad_out is NULL");
  if ((reinterpret_cast<uintptr_t>(feats) | reinterpret_cast<uintptr_t>(grad_out)) & 15)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "feats and grad_out must be 16-byte aligned");
  if (ws > 0 && !workspace) return set_error(SUBMCONV_ERR_INVALID_ARG, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(grad_w) | reinterpret_cast<uintptr_t>(workspace)) & 15)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "grad_w and workspace must be 16-byte aligned");
  int dev = -1;
  SUBMCONV_HIP_CHECK(hipGetDevice(&dev));
  if (dev != m.device)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "the map is on device %d, the current device is %d",
                     m.device, dev);
  const _Float16* f = reinterpret_cast<const _Float16*>(feats);
  const _Float16* g = reinterpret_cast<const _Float16*>(grad_out);
  float* part = static_cast<float*>(workspace);
  if (ws > 0) {
    // the MFMA kernels address rows and lists through 32-bit buffer offsets
    constexpr int64_t kMax = (int64_t{1} << 31) - 64;
    if (m.n * cin * 2 > kMax || m.n * cout * 2 > kMax || (m.active_pairs + 1) * 8 > kMax)
      return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE,
                       "%lld rows x (%d, %d) channels, %lld pairs: features, gradients or lists "
                       "reach 2 GiB, the weight-gradient kernel's 32-bit buffer offsets",
                       static_cast<long long>(m.n), cin, cout,
                       static_cast<long long>(m.active_pairs));
    const int64_t mb = max_blocks;
    if (const int64_t sb = staged_wgrad_blocks(m, ksize, cin, cout); sb > 0 && sb * K <= mb)
      return backward_weight_staged(m, cin, cout, f, g, part, grad_w, stream);
    switch (cin) {
      case 32: return dispatch_w<32>(m, K, cout, f, g, part, grad_w, mb, stream);
      case 64: return dispatch_w<64>(m, K, cout, f, g, part, grad_w, mb, stream);
      case 96: return dispatch_w<96>(m, K, cout, f, g, part, grad_w, mb, stream);
      case 128: return dispatch_w<128>(m, K, cout, f, g, part, grad_w, mb, stream);
      case 160: return dispatch_w<160>(m, K, cout, f, g, part, grad_w, mb, stream);
      case 192: return dispatch_w<192>(m, K, cout, f, g, part, grad_w, mb, stream);
      case 224: return dispatch_w<224>(m, K, cout, f, g, part, grad_w, mb, stream);
      case 256: return dispatch_w<256>(m, K, cout, f, g, part, grad_w, mb, stream);
      default: break;
    }
  }
  const int64_t items = static_cast<int64_t>(K) * cin * (cout / 8);
  k_bwd_weight_valu<<<static_cast<unsigned>((items + 255) / 256), 256, 0, stream>>>(
      K == kTaps3 ? m.nbr : nullptr, m.order, m.n, K, f, g, cin, cout, grad_w);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

}  // namespace
}  // namespace submconv

using namespace submconv;

extern "C" int64_t submconv_backward_weight_workspace_bytes(submconv_map_t map, int32_t cin,
                                                            int32_t cout, int32_t ksize) {
  const int st = check_weight_args(map, cin, cout, ksize);
  if (st != SUBMCONV_OK) return st;
  return workspace_bytes(map->m, cin, cout, ksize, INT64_MAX);
}

extern "C" int submconv_backward_weight(submconv_map_t map, const uint16_t* feats,
                                        const uint16_t* grad_out, float* grad_w, void* workspace,
                                        int32_t cin, int32_t cout, int32_t ksize,
                                        hipStream_t stream) {
  clear_error();
  const int st = check_weight_args(map, cin, cout, ksize);
  if (st != SUBMCONV_OK) return st;
  const int64_t ws = workspace_bytes(map->m, cin, cout, ksize, INT64_MAX);
  return backward_weight_impl(map->m, feats, grad_out, grad_w, workspace, ws, INT64_MAX, cin, cout,
                              ksize, stream);
}

// This device's address of `scratch`, looked up once per device (on the
// entry point's first call there, with that device current) and kept.
static int scratch_address(int dev, void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    SUBMCONV_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    addr[dev] = p;
  }
  *out = addr[dev];
  return SUBMCONV_OK;
}

extern "C" int submconv_backward_weight_noalloc(submconv_map_t map, const uint16_t* feats,
                                                const uint16_t* grad_out, float* grad_w,
                                                int32_t cin, int32_t cout, int32_t ksize,
                                                hipStream_t stream) {
  clear_error();
  const int st = check_weight_args(map, cin, cout, ksize);
  if (st != SUBMCONV_OK) return st;
  const Map& m = map->m;
  int dev = -1;
  SUBMCONV_HIP_CHECK(hipGetDevice(&dev));
  if (dev != m.device)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "the map is on device %d, the current device is %d",
                     m.device, dev);
  void* ws_ptr = nullptr;
  const int sa = scratch_address(dev, &ws_ptr);
  if (sa != SUBMCONV_OK) return sa;
  // as many workgroups' partials as the static workspace holds (longer runs
  // per workgroup than the allocating entry point when they do not all fit)
  const int64_t max_blocks =
      static_cast<int64_t>(kNoAllocScratchBytes / (static_cast<size_t>(cin) * cout * sizeof(float)));
  const int64_t ws = workspace_bytes(m, cin, cout, ksize, max_blocks);
  if (ws > static_cast<int64_t>(kNoAllocScratchBytes))
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE,
                     "the weight gradient needs %lld bytes of partials, the static workspace "
                     "holds %zu", static_cast<long long>(ws), kNoAllocScratchBytes);
  return backward_weight_impl(m, feats, grad_out, grad_w, ws_ptr, ws, max_blocks, cin, cout, ksize,
                              stream);
}

extern "C" int submconv_backward_bias(const uint16_t* grad_out, int64_t n, int32_t cout,
                                      float* grad_b, hipStream_t stream) {
  clear_error();
  if (n < 0 || cout <= 0 || cout % 8 || cout > 1024)
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "n = %lld, Cout = %d", (long long)n, cout);
  if (!grad_b || (n > 0 && !grad_out)) return set_error(SUBMCONV_ERR_INVALID_ARG, "NULL pointer");
  if (reinterpret_cast<uintptr_t>(grad_out) & 15)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "grad_out must be 16-byte aligned");
  k_bwd_bias<<<static_cast<unsigned>(cout / 8), 256, 0, stream>>>(
      reinterpret_cast<const _Float16*>(grad_out), n, cout, grad_b);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}
