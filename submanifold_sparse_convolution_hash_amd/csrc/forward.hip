// SubMConv3d forward on gfx950: a fused, output-stationary gather-GEMM.
//
// out[i] = bias + sum_k feats[nbr[k][i]] @ W[k] is the fused-tap product
// [N, K^3*Cin] x [K^3*Cin, Cout] of the trellis_sparse_mlx README
// ("Performance": one matmul over all taps instead of 2*K^3 dispatches, and a
// cached gather index). The accumulator stays fp32 and the tile operands are
// fp16 or bf16 (the mixed-precision shape of the "Fixed" list of the
// trellis-mac issue #1 thread).
//
// A unit of work is one tile of 256 output rows (in the map's processing
// order) x COUT_T output columns; nothing is shared between units and there
// are no atomics:
//   * The map holds, per tile, the neighbours of every tap compacted into a
//     list of {neighbour row, row in tile}; the tile's steps are the 32-row
//     groups of those lists (the centre tap first, covering every row), so an
//     absent neighbour costs nothing.
//   * A step gathers its 32 feature rows into LDS (16-byte loads, XOR
//     swizzled), multiplies them on v_mfma_f32_32x32x16_f16 (or _bf16) with
//     the tap's weights and adds the 32 x COUT_T result to an fp32 accumulator
//     tile in LDS. Rows are unique within a group and a wave's columns are
//     its own, so the read-modify-write needs no atomics.
//   * k_fwd_pp gives each 32-column block two waves that take the groups in
//     turn, and is persistent: each workgroup walks a run of units with its
//     pipeline running on across them. 256 input channels run as two passes
//     of 128 over each unit. The pipeline is software pipelined with rings of
//     register buffers unrolled to static indices, and ends every step with
//     an LDS-only fence and barrier.
//   * Epilogue: bias in fp32, one rounding (round to nearest even), 16-byte
//     row stores at the caller's row.
#include <algorithm>
#include <atomic>
#include <climits>
#include <mutex>
#include <type_traits>
#include <utility>

#include "submconv_internal.h"

namespace submconv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

// 16-bit element types: rows and fragments move as opaque 16-byte chunks
// (half8); only the MFMA and the final rounding depend on the type.
template <bool IS_BF16>
__device__ __forceinline__ _Float16 round16(float v) {
  if constexpr (IS_BF16)
    return __builtin_bit_cast(_Float16, static_cast<__bf16>(v));  // round to nearest even
  else
    return static_cast<_Float16>(v);  // round to nearest even
}
template <bool IS_BF16>
__device__ __forceinline__ float widen16(_Float16 v) {
  if constexpr (IS_BF16)
    return static_cast<float>(__builtin_bit_cast(__bf16, v));
  else
    return static_cast<float>(v);
}

constexpr int kMaxChannels = 1024;
// mean groups of 32 entries per off-centre position and tile from which a
// map counts as dense (64-row groups at Cin <= 64)
constexpr int kDenseGroups = 3;

__device__ __forceinline__ int excl_scan_wave(int v, int lane) {
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x - v;
}

// Buffer resource over [base, base + bytes): loads at offsets >= bytes return
// zeros without touching memory, which lets masked lanes and skipped loads
// issue the same instructions as live ones (no branches, static wait counts).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
constexpr uint32_t kOob = 0x80000000u;  // an offset past every buffer (< 2 GiB)

__device__ __forceinline__ half8 bload_h8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ int bload_i1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Epilogue of the MFMA kernel: the tile's fp32 accumulator rows (float4
// chunk q of row r at r*NQ + (q ^ (r % NQ))) plus the bias, rounded once to
// fp16 (round to nearest even) and stored at the caller's row. Thread tid
// takes 8 columns c8 = tid % C8 of rows tid / C8 + RPI k. The loop is
// instantiated per presence of bias and order, so that the common case
// issues no vector loads (a wait for one would also wait for the next unit's
// loads already in flight). The outputs are not read again here: streaming
// (non-temporal) stores.
template <int COUT_T, int NT, bool K3, bool IS_BF16, int M>
__device__ __forceinline__ void store_tile(const float4v* acc, int rows_here, int tid,
                                           const float* __restrict__ bias, int c0,
                                           const int32_t* __restrict__ order, int64_t t0,
                                           _Float16* __restrict__ out, int cout) {
  constexpr int NQ = COUT_T / 4;
  constexpr int C8 = COUT_T / 8;
  constexpr int RPI = NT / C8;  // rows per pass
  static_assert(NT % C8 == 0 && M % RPI == 0, "epilogue split");
  const int c8 = tid % C8;
  const int r0 = tid / C8;
  auto body = [&](auto hb, auto ho) {
    constexpr bool HB = decltype(hb)::value, HO = decltype(ho)::value;
    float4v b0 = {0.f, 0.f, 0.f, 0.f}, b1 = {0.f, 0.f, 0.f, 0.f};
    if constexpr (HB) {
      b0 = *reinterpret_cast<const float4v*>(bias + c0 + 8 * c8);
      b1 = *reinterpret_cast<const float4v*>(bias + c0 + 8 * c8 + 4);
    }
#pragma unroll 2
    for (int k = 0; k < M / RPI; ++k) {
      const int r = r0 + RPI * k;
      if (r < rows_here) {
        const int q0 = 2 * c8, q1 = 2 * c8 + 1;
        const float4v a = acc[r * NQ + (q0 ^ (r & (NQ - 1)))];
        const float4v b = acc[r * NQ + (q1 ^ (r & (NQ - 1)))];
        half8 hv;
        hv[0] = round16<IS_BF16>(a[0] + b0[0]);
        hv[1] = round16<IS_BF16>(a[1] + b0[1]);
        hv[2] = round16<IS_BF16>(a[2] + b0[2]);
        hv[3] = round16<IS_BF16>(a[3] + b0[3]);
        hv[4] = round16<IS_BF16>(b[0] + b1[0]);
        hv[5] = round16<IS_BF16>(b[1] + b1[1]);
        hv[6] = round16<IS_BF16>(b[2] + b1[2]);
        hv[7] = round16<IS_BF16>(b[3] + b1[3]);
        const int64_t orow = HO ? order[t0 + r] : t0 + r;
        __builtin_nontemporal_store(hv,
                                    reinterpret_cast<half8*>(out + orow * cout + c0 + 8 * c8));
      }
    }
  };
  using T = std::true_type;
  using F = std::false_type;
  if (bias) {
    if (K3 && order)
      body(T{}, T{});
    else
      body(T{}, F{});
  } else {
    if (K3 && order)
      body(F{}, T{});
    else
      body(F{}, F{});
  }
}

typedef float float16v __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// Two-wave (ping-pong) MFMA kernel
// ---------------------------------------------------------------------------
//
// A workgroup owns a unit's 256 x COUT_T fp32 accumulator in LDS. Each
// 32-column block has two waves that take the groups of the tile in turn
// (group: 32 entries of one position's list, or 64 on dense maps). In step f the
// wave of parity f % 2 multiplies group f and adds it to its rows of the LDS
// accumulator (the old rows are requested before the MFMAs, so their latency
// overlaps them), while its partner reads the B fragments of group f+1 and
// requests the row indices of group f+1 and the weights of group f+3. With
// two waves per SIMD the instruction stream of a step has two issuers and one
// wave's MFMAs overlap the other's LDS and address work. Consecutive groups
// may update the same rows; their updates are in consecutive steps, ordered
// by the step barrier. All waves share the gathering of feature rows.
//
// The grid is as many workgroups as the compute units hold at once (one per
// CU when the 128-column accumulator fills the LDS), and each walks every
// wpx-th unit of its XCD's run. The steps of successive units form one
// stream: the lookahead reads the next unit's schedule, so that unit's
// entries, rows, weights and first gathered groups are in flight while the
// current one finishes and writes its outputs, and only the first unit pays
// for filling the pipeline.

template <int CIN, int COUT_T, bool K3, int GR_ = 32, int M_ = kTileRows>
struct CfgPP {
  static constexpr int M = M_;               // accumulator rows: the map's tiles have at most M
  static constexpr int GR = GR_;             // rows per group: 32, or 64 for dense maps
  static constexpr int NRB = GR / 32;        // 32-row MFMA blocks per group
  static constexpr int NC = COUT_T / 32;     // column blocks
  // waves sharing a group's row blocks: narrow tiles of 64-row groups split
  // them, so that a step's work is spread over more waves
  static constexpr int RS = (GR == 64 && COUT_T <= 64) ? 2 : 1;
  static constexpr int NRBW = NRB / RS;      // row blocks per wave
  static constexpr int NW = 2 * NC * RS;     // waves: two per column block and row split
  static constexpr int NT = 64 * NW;
  static constexpr int KS = CIN / 16;
  static constexpr int NQ = COUT_T / 4;
  static constexpr int RC = CIN / 8;
  static constexpr int GCH = GR * RC;
  static constexpr int CPT = GCH >= NT ? GCH / NT : 1;
  static constexpr int NLOAD = GCH >= NT ? NT : GCH;
  static constexpr int NCG = M / GR;         // steps of the centre
  static constexpr int BR = (4 - NCG % 4) % 4;  // steps after them up to a multiple of 4
  static constexpr int LB = 4;               // chunks requested LB steps before the multiply
  static constexpr int LE = 2;               // entries LE steps before their chunks
  static_assert(CIN % 32 == 0 && CIN <= 128, "CIN");
  static_assert(COUT_T % 32 == 0 && COUT_T <= 128, "COUT_T");
  static_assert(GCH % NT == 0 || NT % GCH == 0, "chunk split");
  static_assert(M % GR == 0 && LB <= 4 && LE < 4, "schedule");
  static_assert(GR == 32 || GR == 64, "GR");
  static_assert(M * COUT_T * 4 + 2 * GCH * 16 <= 163840, "LDS");
};

// NP > 1 splits the channels of each feature row into NP passes of CIN (the
// 256-channel layer runs as two 128-channel passes over each unit): a unit
// then takes NP runs of its schedule into the same accumulator, the first
// pass's centre steps writing it and the last pass writing the outputs. Pass
// p takes K steps p KS .. p KS + KS - 1 of the row's MFMA K order (channels
// h CIN_T/2 + 8 st + j of lane half h), so the weights keep their layout.
template <int CIN, int COUT_T, bool K3, bool IS_BF16, int GR_, int NP = 1, int M_ = kTileRows>
__global__ __launch_bounds__((CfgPP<CIN, COUT_T, K3, GR_, M_>::NT)) void k_fwd_pp(
    const int2* __restrict__ ent, const int32_t* __restrict__ tile_off,
    const uint16_t* __restrict__ tile_cnt, const int32_t* __restrict__ walk,
    const int32_t* __restrict__ order, int64_t n, const _Float16* __restrict__ feats,
    const _Float16* __restrict__ wp, const float* __restrict__ bias, _Float16* __restrict__ out,
    int cout, int n_tiles, int n_ct, int tiles_per_xcd, int n_pairs, int tile_rows) {
  // tile_rows: the map's rows per tile, at most M (the LDS accumulator's
  // rows); walk: the tile at each position of an XCD's run, or nullptr for
  // tile i at position i
  using C = CfgPP<CIN, COUT_T, K3, GR_, M_>;
  constexpr int M = C::M, GR = C::GR, NRBW = C::NRBW, KS = C::KS, RC = C::RC;
  constexpr int LB = C::LB, LE = C::LE, CPT = C::CPT, NCG = C::NCG, BR = C::BR;
  constexpr int CIN_T = CIN * NP, KST = KS * NP;  // channels and K steps of a whole row
  __shared__ float4v acc[M * C::NQ];
  __shared__ half8 bt[2][C::GCH];

  // Persistent: the workgroups of an XCD (blockIdx % 8) walk that XCD's
  // contiguous run of units (row tile, column tile), so neighbouring tiles,
  // which gather the same feature rows, share an L2; each workgroup takes
  // every wpx-th unit.
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int j0 = bid >> 3;
  const int wpx = static_cast<int>(gridDim.x >> 3);
  const int units = tiles_per_xcd * n_ct;
  // units past the end come last in a workgroup's walk; one that starts
  // there has nothing to do
  if (j0 >= units || xcd * tiles_per_xcd + j0 / n_ct >= n_tiles) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int par = w / (C::NC * C::RS);  // the parity of the groups this wave multiplies
  const int wr = w - par * C::NC * C::RS;
  const int wc = wr % C::NC;            // its column block
  const int rb0 = (wr / C::NC) * NRBW;  // and its first row block

  // ---- per-unit schedules ----
  // The workgroup's s-th run of a schedule: unit j0 + (s / NP) wpx, pass s % NP.
  struct Raw {
    int cnt, ent0, tile, ct, pass;
  };
  auto raw_of = [&](int s) -> Raw {  // issue the loads of run s's counts
    Raw r{0, 0, -1, 0, s % NP};
    const int u = j0 + (s / NP) * wpx;
    const int tl = u / n_ct;
    const int pos = xcd * tiles_per_xcd + tl;
    if (u < units && tl < tiles_per_xcd && pos < n_tiles) {
      const int tile = walk ? walk[pos] : pos;
      r.tile = tile;
      r.ct = u - tl * n_ct;
      if (K3) {
        if (lane < kTaps3) r.cnt = tile_cnt[static_cast<int64_t>(tile) * kTaps3 + lane];
        r.ent0 = tile_off[tile];
      }
    }
    return r;
  };
  // One unit's schedule in lanes 0..31. For processing position p < 27 (the
  // centre first): cnt entries, the first at off (in the whole list, or the
  // row in the tile for a 1x1x1 kernel), processed from step gs on (the
  // centre in NCG steps, then each position in steps of GR entries). Lane 27
  // is an empty position at step F, where the unit's steps end; the unit
  // takes Fp steps: F rounded up to a multiple of 4, so that step residues
  // mod 4 carry over to the next unit, and to at least the centre's steps
  // rounded up and kMinSteps. The pipeline looks LB + LE steps ahead, and the
  // schedule holds two units: a unit's last steps must not look past the
  // next one, even when that one is all centre (64-row groups take the centre
  // in 4 steps). Lanes 28..31 start at no step. wb is the byte offset of the
  // position's weights for the unit's column tile.
  constexpr int kMinSteps = (LB + LE + 3) & ~3;
  struct Half {
    int cnt, off, gs, wb;  // per lane
    int F, Fp, c0, rows_here, pass;
    int64_t t0;
  };
  auto half_of = [&](const Raw& r) -> Half {  // the counts have arrived
    Half hf;
    const bool live = r.tile >= 0;
    hf.t0 = static_cast<int64_t>(live ? r.tile : 0) * tile_rows;
    hf.rows_here = live ? static_cast<int>(n - hf.t0 < tile_rows ? n - hf.t0 : tile_rows) : 0;
    hf.c0 = r.ct * COUT_T;
    hf.cnt = K3 ? (live ? r.cnt : 0) : (lane == 0 ? hf.rows_here : 0);
    hf.off = excl_scan_wave(hf.cnt, lane) + (K3 ? __builtin_amdgcn_readfirstlane(r.ent0) : 0);
    const int ng = (lane >= 1 && lane < kTaps3) ? (hf.cnt + GR - 1) / GR : 0;
    const int gs = NCG + excl_scan_wave(ng, lane);
    hf.F = live ? __builtin_amdgcn_readlane(gs, kTaps3) : 0;
    hf.Fp = live ? max(NCG + BR + ((max(hf.F - NCG - BR, 0) + 3) & ~3), kMinSteps) : 0;
    hf.gs = lane == 0 ? 0 : (lane <= kTaps3 ? gs : INT_MAX);
    hf.wb = (((K3 ? tap_at(lane & 31) * (cout / 32) : 0) + r.ct * (COUT_T / 32)) * KST +
             r.pass * KS) * 1024;
    hf.pass = r.pass;
    return hf;
  };
  struct Grp {
    int start, cnt, wb, pass;
    int64_t t0;
  };
  // The stream's schedule: the current unit a in lanes 0..31, the next unit b
  // in lanes 32..63 with its steps counted on from a's last.
  // Per lane: gs, the first step of the position; offg = off - GR gs, so
  // that step f of the position starts at entry offg + GR f; end = off + cnt;
  // and wb.
  int s_gs, s_offg, s_end, s_wb;
  auto join = [&](const Half& a, const Half& b) {
    const int bc = __shfl_xor(b.cnt, 32);
    const int bo = __shfl_xor(b.off, 32);
    const int bg = __shfl_xor(b.gs, 32);
    const int bw = __shfl_xor(b.wb, 32);
    const bool lo = lane < 32;
    const int cnt = lo ? a.cnt : bc;
    const int off = lo ? a.off : bo;
    s_gs = lo ? a.gs : (bg == INT_MAX ? INT_MAX : bg + a.Fp);
    s_offg = s_gs == INT_MAX ? 0 : off - GR * s_gs;
    s_end = off + cnt;
    s_wb = lo ? a.wb : bw;
  };
  // group of step f: the last lane whose position starts at or before f
  auto group_at = [&](const Half& a, const Half& b, int f) -> Grp {
    const uint64_t m = __ballot(s_gs <= f);
    const int p = 63 - __builtin_clzll(m);
    Grp g;
    g.start = __builtin_amdgcn_readlane(s_offg, p) + GR * f;
    const int c = __builtin_amdgcn_readlane(s_end, p) - g.start;
    g.cnt = c < GR ? c : GR;  // <= 0 past the position's entries
    g.wb = __builtin_amdgcn_readlane(s_wb, p);
    g.t0 = p < 32 ? a.t0 : b.t0;
    g.pass = NP == 1 ? 0 : (p < 32 ? a.pass : b.pass);
    return g;
  };

  const __amdgpu_buffer_rsrc_t rf = make_rsrc(feats, static_cast<uint32_t>(n * CIN_T * 2));
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(wp, static_cast<uint32_t>((K3 ? kTaps3 : 1) * CIN_T * cout * 2));
  const __amdgpu_buffer_rsrc_t re = make_rsrc(ent, static_cast<uint32_t>(n_pairs + 1) * 8u);
  const uint32_t e_none = static_cast<uint32_t>(n_pairs) * 8u;

  // ---- loader role (all waves) ----
  const bool loader = tid < C::NLOAD;
  int lrow[CPT], lpos[CPT];
  uint32_t lcol[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + C::NT * i;
    lrow[i] = c / RC;
    const int lc = c % RC;
    // byte offset in the row of local chunk lc (K steps lc % KS of lane half
    // lc / KS) in pass 0
    lcol[i] = static_cast<uint32_t>(((lc / KS) * (CIN_T / 16) + lc % KS) * 16);
    lpos[i] = lrow[i] * RC + (lc ^ (lrow[i] & (RC - 1)));
  }
  // the feature row of each of this thread's chunks of group g (-1: none;
  // only the entries' first word, the neighbour's row, is read), and (ep)
  // the pass the chunks are for
  auto load_entries = [&](const Grp& g, int (&E)[CPT], int& ep) {
    ep = g.pass;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const bool live = loader && lrow[i] < g.cnt;
      if (K3)
        E[i] = bload_i1(re, live ? static_cast<uint32_t>(g.start + lrow[i]) * 8u : e_none);
      else
        E[i] = live ? static_cast<int>(g.t0) + g.start + lrow[i] : -1;
    }
  };
  auto load_chunks = [&](const int (&E)[CPT], int ep, half8 (&D)[CPT]) {
    const uint32_t pc = NP == 1 ? 0u : static_cast<uint32_t>(ep * KS * 16);
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      D[i] = bload_h8(rf, E[i] >= 0 ? static_cast<uint32_t>(E[i]) * (CIN_T * 2) + pc + lcol[i]
                                    : kOob);
  };
  auto store_chunks = [&](int slot, const half8 (&D)[CPT]) {
    if (loader) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) bt[slot][lpos[i]] = D[i];
    }
  };
  // row in tile of this lane's slot in each 32-row block of group g (-1: none)
  auto load_row = [&](const Grp& g, int (&R)[NRBW]) {
#pragma unroll
    for (int rb = 0; rb < NRBW; ++rb) {
      const int sl = (lane & 31) + 32 * (rb0 + rb);
      if (K3)
        R[rb] = bload_i1(re, (sl < g.cnt ? static_cast<uint32_t>(g.start + sl) * 8u : e_none) + 4u);
      else
        R[rb] = sl < g.cnt ? g.start + sl : -1;
    }
  };

  // ---- MFMA role: the two waves of a block own its 32 output columns ----
  // v_mfma_f32_32x32x16_f16 computes out^T for 32 rows of the group: A =
  // weights (lane: column lane%32, K steps st of lane half lane/32, 8
  // channels each), B = gathered rows (lane: slot lane%32, the same
  // channels), D: lane holds slot lane%32 and columns 8*a + 4*(lane/32) + b
  // in register 4*a + b.
  const int s32 = lane & 31;
  const int h = lane >> 5;
  const int qw = wc * 8;
  auto load_a = [&](const Grp& g, half8 (&A)[KS]) {
    const uint32_t base = static_cast<uint32_t>(g.wb + wc * KST * 1024 + lane * 16);
    // one select; the K-step offsets fold into the loads' immediate offsets
    const uint32_t b = g.cnt > 0 ? base : kOob;
#pragma unroll
    for (int st = 0; st < KS; ++st) A[st] = bload_h8(rw, b + st * 1024);
  };
  int boff[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    const int lc = h * (CIN / 16) + st;
    boff[st] = s32 * RC + (lc ^ (s32 & (RC - 1)));
  }
  // B fragments of this wave's 32-row blocks (block rb: rows 32 rb.., the
  // same swizzle since 32 rb is a multiple of RC)
  auto read_b = [&](int slot, half8 (&B)[NRBW][KS]) {
#pragma unroll
    for (int rb = 0; rb < NRBW; ++rb)
#pragma unroll
      for (int st = 0; st < KS; ++st) B[rb][st] = bt[slot][boff[st] + 32 * (rb0 + rb) * RC];
  };
  auto multiply = [&](const half8 (&A)[KS], const half8 (&B)[KS]) {
    float16v d = {};
#pragma unroll
    for (int st = 0; st < KS; ++st)
      if constexpr (IS_BF16)
        d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, A[st]),
                                                    __builtin_bit_cast(bf16x8, B[st]), d, 0, 0, 0);
      else
        d = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[st], B[st], d, 0, 0, 0);
    return d;
  };
  // chunk qw + 2a + h of row r sits at r*NQ + ((qw + 2a + h) ^ (r % NQ));
  // qw is a multiple of 8 and 2a + h < 8, so that is a0 ^ 2a with a0 the
  // slot of a = 0
  auto acc_at = [&](int a0, int a) { return a0 ^ (2 * a); };
  auto acc_row = [&](int r) { return r * C::NQ + ((qw + h) ^ (r & (C::NQ - 1))); };
  auto read_old = [&](int r, float4v (&old)[4]) {
    if (r >= 0) {
      const int a0 = acc_row(r);
#pragma unroll
      for (int a = 0; a < 4; ++a) old[a] = acc[acc_at(a0, a)];
    }
  };
  auto write_acc = [&](int r, bool centre, const float4v (&old)[4], const float16v& d) {
    if (r >= 0) {
      const int a0 = acc_row(r);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float4v v = {d[4 * a], d[4 * a + 1], d[4 * a + 2], d[4 * a + 3]};
        acc[acc_at(a0, a)] = centre ? v : old[a] + v;
      }
    }
  };
  auto lds_barrier = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  // ---- pipeline ----
  // The steps of this workgroup's units form one stream: a step's lookahead
  // past the end of the current unit reads the next unit's schedule, so the
  // next unit's entries, rows, weights and first gathered groups are in
  // flight while the current one finishes and writes its epilogue.
  // Loader: group g's entries in step g-LB-LE, chunks in step g-LB, stored
  // to slot g%2 in step g-2. A wave multiplies the groups g of its parity:
  // weights requested in step g-3 (set (g/2)%2), B fragments and row indices
  // in step g-1; in step g it multiplies g and adds it to its rows.
  // The pipeline is instantiated once per parity, so that every wave's roles,
  // and with them its memory-counter waits, are static.
  auto run = [&](auto parc) {
    constexpr int PAR = decltype(parc)::value;
    int s = 0;
    Half cur = half_of(raw_of(0));
    Half nxt = half_of(raw_of(1));
    Raw raw = raw_of(2);
    join(cur, nxt);
    auto grp = [&](int f) -> Grp { return group_at(cur, nxt, f); };

    int E[4][CPT];
    int EP[4];
    half8 D[4][CPT];
    int RW[2][NRBW];
    half8 AW[2][KS];
    half8 BF[NRBW][KS];
#pragma unroll
    for (int g = 0; g < LB; ++g) load_entries(grp(g), E[g % 4], EP[g % 4]);
#pragma unroll
    for (int g = 0; g < LB; ++g) load_chunks(E[g % 4], EP[g % 4], D[g % 4]);
#pragma unroll
    for (int g = LB; g < LB + LE; ++g) load_entries(grp(g), E[g % 4], EP[g % 4]);
    if (PAR == 0) {
      load_a(grp(0), AW[0]);
      load_a(grp(2), AW[1]);
      load_row(grp(0), RW[0]);
    } else {
      load_a(grp(1), AW[0]);
    }
    store_chunks(0, D[0]);
    store_chunks(1, D[1]);
    lds_barrier();
    if (PAR == 0) read_b(0, BF);
    lds_barrier();

    // step f of the current unit; i = f mod 4
    auto step = [&](int f, auto ic, auto cc) {
      constexpr int i = decltype(ic)::value;
      constexpr bool centre_step = decltype(cc)::value;
      store_chunks(i & 1, D[(i + 2) % 4]);
      if constexpr (PAR == (i & 1)) {
        // multiply group f and add it to the accumulator; the old rows are
        // requested before the MFMAs so that their latency overlaps them.
        // This chain ends the step, so the wave issues ahead of its partner
        // (whose B-fragment reads would otherwise queue in front in LDS).
        float4v old[NRBW][4];
        __builtin_amdgcn_s_setprio(3);
        // the centre steps of the first pass write the accumulator
        const bool first = centre_step && (NP == 1 || cur.pass == 0);
        if (!first) {
#pragma unroll
          for (int rb = 0; rb < NRBW; ++rb) read_old(RW[(i >> 1) & 1][rb], old[rb]);
        }
        if (centre_step || f < cur.F) {
#pragma unroll
          for (int rb = 0; rb < NRBW; ++rb) {
            const float16v d = multiply(AW[(i >> 1) & 1], BF[rb]);
            write_acc(RW[(i >> 1) & 1][rb], first, old[rb], d);
          }
        }
        __builtin_amdgcn_s_setprio(0);
        load_chunks(E[(i + LB) % 4], EP[(i + LB) % 4], D[(i + LB) % 4]);
        load_entries(grp(f + LB + LE), E[(i + LB + LE) % 4], EP[(i + LB + LE) % 4]);
      } else {
        // prepare this wave's next group, f+1. Its rows are requested
        // first: the memory counter completes in order, so the multiply's
        // wait for them then leaves every later load of this step in flight.
        load_row(grp(f + 1), RW[((i + 1) >> 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        read_b((i + 1) & 1, BF);
        load_a(grp(f + 3), AW[((i + 3) >> 1) & 1]);
        load_chunks(E[(i + LB) % 4], EP[(i + LB) % 4], D[(i + LB) % 4]);
        load_entries(grp(f + LB + LE), E[(i + LB + LE) % 4], EP[(i + LB + LE) % 4]);
      }
      lds_barrier();
    };
    while (true) {
      [&]<int... I>(std::integer_sequence<int, I...>) {
        (step(I, std::integral_constant<int, I % 4>{}, std::true_type{}), ...);
      }(std::make_integer_sequence<int, NCG>{});
      // steps up to a multiple of 4, so that the ring indices below are
      // static and carry over to the next unit
      [&]<int... I>(std::integer_sequence<int, I...>) {
        (step(NCG + I, std::integral_constant<int, (NCG + I) % 4>{}, std::false_type{}), ...);
      }(std::make_integer_sequence<int, BR>{});
      for (int f0 = NCG + BR; f0 < cur.Fp; f0 += 4) {
        [&]<int... I>(std::integer_sequence<int, I...>) {
          (step(f0 + I, std::integral_constant<int, I>{}, std::false_type{}), ...);
        }(std::make_integer_sequence<int, 4>{});
      }
      // the last step's barrier made every update visible
      if (NP == 1 || cur.pass == NP - 1)
        store_tile<COUT_T, C::NT, K3, IS_BF16, M>(acc, cur.rows_here, tid, bias, cur.c0, order,
                                                  cur.t0, out, cout);
      if (nxt.F == 0) break;
      lds_barrier();  // the epilogue's reads are done before the next centre writes
      cur = nxt;
      nxt = half_of(raw);
      join(cur, nxt);
      ++s;
      raw = raw_of(s + 2);
    }
  };
  if (par == 0)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, 1>{});
}

// ---------------------------------------------------------------------------
// VALU kernel for channel counts the MFMA tiles do not cover (multiples of 8)
// ---------------------------------------------------------------------------

// One thread per (row, output column): consecutive threads take consecutive
// columns of a row, so the row's neighbour indices and feature chunks are
// shared loads and the weight loads and output stores are coalesced. The
// neighbour indices are loaded first, all at once, and the taps are unrolled
// with a select instead of a branch, so that the loads of successive taps
// are in flight together (a tiny layer is otherwise a chain of load
// latencies). The weights are read as the caller holds them: W_t[k][ci][co]
// = W[k][ci][co], or for the input gradient (GRAD) the flipped, transposed
// W[K-1-k][co][ci] of the layer's W [K][cout][cin].
template <bool K3, bool IS_BF16, bool GRAD>
__global__ __launch_bounds__(256) void k_fwd_valu(
    const int32_t* __restrict__ nbr, const int32_t* __restrict__ order, int64_t n,
    const _Float16* __restrict__ feats, const _Float16* __restrict__ w,
    const float* __restrict__ bias, _Float16* __restrict__ out, int cin, int cout) {
  constexpr int K = K3 ? kTaps3 : 1;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < n * cout;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t t = idx / cout;
    const int o = static_cast<int>(idx - t * cout);
    float a = bias ? bias[o] : 0.f;
    int js[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
      js[k] = K3 ? nbr[static_cast<int64_t>(k) * n + t] : static_cast<int>(t);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      // an absent neighbour reads row 0 and leaves the sum unchanged
      const bool live = js[k] >= 0;
      const half8* f8 =
          reinterpret_cast<const half8*>(feats + static_cast<int64_t>(live ? js[k] : 0) * cin);
      // W_t[k][ci][o] = wk[ci * ws]
      const _Float16* wk = GRAD ? w + (static_cast<int64_t>(K - 1 - k) * cout + o) * cin
                                : w + static_cast<int64_t>(k) * cin * cout + o;
      const int64_t ws = GRAD ? 1 : cout;
      for (int c8 = 0; c8 < cin / 8; ++c8) {
        const half8 fv = f8[c8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = fmaf(widen16<IS_BF16>(fv[e]),
                               widen16<IS_BF16>(wk[static_cast<int64_t>(8 * c8 + e) * ws]), a);
          a = live ? v : a;
        }
      }
    }
    const int64_t orow = (K3 && order) ? order[t] : t;
    out[orow * cout + o] = round16<IS_BF16>(a);
  }
}

// ---------------------------------------------------------------------------
// weight preparation
// ---------------------------------------------------------------------------

// Weights of the forward being prepared, W_t[k][ci][co] for a forward with
// cin x cout channels: W itself, or for the input gradient the flipped,
// transposed kernel W_t[k][ci][co] = W[K-1-k][co][ci] of W [K][cout][cin]
// (out[i] gathers feats[c_i + d_k]; its input gradient gathers grad_out at
// c_j - d_k = c_j + d_(K-1-k) through W[k]^T, so the same forward on the same
// map computes it).
__device__ __forceinline__ _Float16 weight_at(const _Float16* __restrict__ W, int K, int cin,
                                              int cout, bool grad, int k, int ci, int co) {
  return grad ? W[(static_cast<int64_t>(K - 1 - k) * cout + co) * cin + ci]
              : W[(static_cast<int64_t>(k) * cin + ci) * cout + co];
}

// MFMA fragment order (v_mfma_f32_32x32x16_f16, weights as the A operand):
// for tap k, 32-column block cb, 16-channel K step st and lane l, 8
// consecutive fp16 values W_t[k][ci][co] with co = 32*cb + (l % 32) and
// ci = (l / 32) * (Cin / 2) + 8*st + j, j = 0..7: one contiguous 1 KiB run per
// (k, cb, st), loaded by a wave with one 16-byte load per lane. One thread
// writes one lane's 8 values (a 16-byte store).
__global__ void k_prepare_mfma(const _Float16* __restrict__ W, int K, int cin, int cout, bool grad,
                               _Float16* __restrict__ wp) {
  // (32-bit index arithmetic: at most 27 x 1024 x 1024 / 8 chunks)
  const uint32_t total8 = static_cast<uint32_t>(K) * cin * cout / 8;
  const uint32_t idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total8) return;
  const uint32_t KS = cin / 16, NCB = cout / 32;
  const int l = static_cast<int>(idx & 63);
  uint32_t rest = idx >> 6;
  const int st = static_cast<int>(rest % KS);
  rest /= KS;
  const int cb = static_cast<int>(rest % NCB);
  const int k = static_cast<int>(rest / NCB);
  const int co = 32 * cb + (l & 31);
  const int ci0 = (l >> 5) * (cin / 2) + 8 * st;
  half8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = weight_at(W, K, cin, cout, grad, k, ci0 + j, co);
  *reinterpret_cast<half8*>(wp + 8 * static_cast<int64_t>(idx)) = v;
}

// Natural order W_t[k][ci][co] (the VALU kernel's layout).
__global__ void k_prepare_plain(const _Float16* __restrict__ W, int K, int cin, int cout, bool grad,
                                _Float16* __restrict__ wp) {
  const int64_t total = static_cast<int64_t>(K) * cin * cout;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int co = static_cast<int>(idx % cout);
  const int ci = static_cast<int>((idx / cout) % cin);
  const int k = static_cast<int>(idx / (static_cast<int64_t>(cout) * cin));
  wp[idx] = weight_at(W, K, cin, cout, grad, k, ci, co);
}

bool use_mfma(int cin, int cout) {
  if (cin == 256) return cout % 128 == 0;
  return (cin == 32 || cin == 64 || cin == 128) && cout % 32 == 0;
}

// The MFMA kernel addresses features and lists through 32-bit buffer
// offsets, with kOob (2 GiB) as the offset of a lane that loads nothing.
constexpr int64_t kMaxBufferBytes = (int64_t{1} << 31) - 64;

// Kernel of a forward: 1 MFMA, 0 VALU, or a negative status.
int kernel_path(int64_t n, int64_t pairs, int cin, int cout, int ksize) {
  if (!use_mfma(cin, cout)) return 0;
  if (n * cin * 2 > kMaxBufferBytes)
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE,
                     "features of %lld rows x %d channels reach 2 GiB, the MFMA kernel's "
                     "32-bit buffer offsets", static_cast<long long>(n), cin);
  if (ksize == 3 && (pairs + 1) * 8 > kMaxBufferBytes)
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE,
                     "%lld active pairs: the per-tile lists reach 2 GiB, the MFMA kernel's "
                     "32-bit buffer offsets", static_cast<long long>(pairs));
  return 1;
}

int check_shape(int32_t ksize, int32_t cin, int32_t cout) {
  if (ksize != 1 && ksize != 3)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "ksize = %d is not 1 or 3", ksize);
  if (cin <= 0 || cout <= 0 || cin % 8 || cout % 8 || cin > kMaxChannels || cout > kMaxChannels)
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE,
                     "Cin = %d, Cout = %d: both must be positive multiples of 8 up to %d", cin,
                     cout, kMaxChannels);
  return SUBMCONV_OK;
}

// compute units per XCD of the current device (MI355X: 256 / 8), cached per
// device
int cus_per_xcd() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 32;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 256;
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    v = std::max(1, cus / 8);
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// workgroups of one instance that a CU holds at once (cached)
template <int CIN, int COUT_T, bool K3, bool IS_BF16, int GR, int NP, int M>
int pp_per_cu() {
  static const int per_cu = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &nb, reinterpret_cast<const void*>(k_fwd_pp<CIN, COUT_T, K3, IS_BF16, GR, NP, M>),
            CfgPP<CIN, COUT_T, K3, GR, M>::NT, 0) != hipSuccess)
      nb = 1;
    return std::max(1, nb);
  }();
  return per_cu;
}

// rounds of the persistent grid: units of an XCD over its workgroups
template <int CIN, int COUT_T, bool K3, bool IS_BF16, int GR, int NP, int M>
int64_t pp_rounds(int64_t n_tiles, int n_ct) {
  const int64_t units_per_xcd = (n_tiles + 7) / 8 * n_ct;
  const int64_t slots = int64_t{cus_per_xcd()} * pp_per_cu<CIN, COUT_T, K3, IS_BF16, GR, NP, M>();
  return (units_per_xcd + slots - 1) / slots;
}

template <int CIN, int COUT_T, bool K3, bool IS_BF16, int GR, int NP = 1, int M = kTileRows>
int launch_pp(const Map& m, const Tiles& T, const _Float16* feats, const _Float16* wp,
              const float* bias, _Float16* out, int cout, hipStream_t stream) {
  if (T.n > (int64_t{1} << 28)) return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "too many rows");
  if (T.rows > M)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "internal: %d tile rows above %d", T.rows, M);
  using C = CfgPP<CIN, COUT_T, K3, GR, M>;
  const int n_tiles = static_cast<int>(T.n);
  const int n_ct = cout / COUT_T;
  const int tiles_per_xcd = (n_tiles + 7) / 8;
  const int n_pairs = static_cast<int>(K3 ? m.active_pairs : 0);
  // persistent: as many workgroups as the CUs hold at once (one per CU when
  // the accumulator fills the LDS, more for narrow column tiles), dealt
  // evenly to the 8 XCDs
  const int per_cu = pp_per_cu<CIN, COUT_T, K3, IS_BF16, GR, NP, M>();
  const int64_t units_per_xcd = int64_t{tiles_per_xcd} * n_ct;
  const int64_t wpx = std::min<int64_t>(units_per_xcd, int64_t{cus_per_xcd()} * per_cu);
  k_fwd_pp<CIN, COUT_T, K3, IS_BF16, GR, NP, M><<<static_cast<unsigned>(8 * wpx), C::NT, 0,
                                                 stream>>>(
      K3 ? T.ent : nullptr, K3 ? T.off : nullptr, K3 ? T.cnt : nullptr, K3 ? T.walk : nullptr,
      K3 ? m.order : nullptr, m.n, feats, wp, bias, out, cout, n_tiles, n_ct, tiles_per_xcd,
      n_pairs, T.rows);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

template <int CIN, int COUT_T, bool K3, bool IS_BF16>
int launch_one(const Map& m, const _Float16* feats, const _Float16* wp, const float* bias,
               _Float16* out, int cout, hipStream_t stream) {
  constexpr int CP = CIN <= 128 ? CIN : 128, NP = CIN <= 128 ? 1 : 2;  // 256 channels: two passes
  static_assert(CIN <= 128 || CIN == 256, "CIN");
  if constexpr (!K3) {
    // a 1x1x1 forward tiles the rows itself
    Tiles rows;
    rows.n = (m.n + kTileRows - 1) / kTileRows;
    return launch_pp<CP, COUT_T, K3, IS_BF16, 32, NP>(m, rows, feats, wp, bias, out, cout, stream);
  } else {
    const int n_ct = cout / COUT_T;
    // dense maps (many groups per position) take 64-row groups: half the
    // steps, each weight load serving two MFMA row blocks. At 128 channels a
    // pass fits the LDS only with 128 columns (exactly 160 KiB); narrower
    // column tiles keep 32-row groups, and two or more workgroups per CU.
    if constexpr (CIN <= 64 || COUT_T == 128) {
      int64_t off_groups = 0;
      for (int q = 1; q < kTaps3; ++q) off_groups += m.tiles.pos_groups[q];
      if (off_groups >= int64_t{kDenseGroups} * (kTaps3 - 1) * m.tiles.n)
        return launch_pp<CP, COUT_T, K3, IS_BF16, 64, NP>(m, m.tiles, feats, wp, bias, out, cout,
                                                         stream);
    }
    // a sparse map's wide tiles (32-row groups) when they fit this layer's
    // workgroups into fewer rounds than 256-row tiles
    if (m.wide.n > 0 &&
        (m.wide_always ||
         pp_rounds<CP, COUT_T, K3, IS_BF16, 32, NP, kTileRowsWide>(m.wide.n, n_ct) <
             pp_rounds<CP, COUT_T, K3, IS_BF16, 32, NP, kTileRows>(m.tiles.n, n_ct)))
      return launch_pp<CP, COUT_T, K3, IS_BF16, 32, NP, kTileRowsWide>(m, m.wide, feats, wp, bias,
                                                                      out, cout, stream);
    return launch_pp<CP, COUT_T, K3, IS_BF16, 32, NP>(m, m.tiles, feats, wp, bias, out, cout,
                                                     stream);
  }
}

template <int CIN, int COUT_T, bool IS_BF16>
int launch_mfma(const Map& m, int ksize, const _Float16* feats, const _Float16* wp,
                const float* bias, _Float16* out, int cout, hipStream_t stream) {
  if (ksize == 1) return launch_one<CIN, COUT_T, false, IS_BF16>(m, feats, wp, bias, out, cout, stream);
  return launch_one<CIN, COUT_T, true, IS_BF16>(m, feats, wp, bias, out, cout, stream);
}

template <int CIN, bool IS_BF16>
int dispatch_cout(const Map& m, int ksize, const _Float16* feats, const _Float16* wp,
                  const float* bias, _Float16* out, int cout, hipStream_t stream) {
  // The LDS holds a 256 x COUT_T fp32 accumulator plus two 32-row groups of
  // Cin channels (at Cin = 256 and 128 columns that is exactly 160 KiB).
  if (cout % 128 == 0) return launch_mfma<CIN, 128, IS_BF16>(m, ksize, feats, wp, bias, out, cout, stream);
  if constexpr (CIN <= 128) {
    if (cout % 64 == 0) return launch_mfma<CIN, 64, IS_BF16>(m, ksize, feats, wp, bias, out, cout, stream);
    return launch_mfma<CIN, 32, IS_BF16>(m, ksize, feats, wp, bias, out, cout, stream);
  }
  return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "internal: no MFMA tile for Cin = %d", CIN);
}

// The forward on weights in the kernel's layout: prepared MFMA fragments
// when the shape takes the MFMA kernel, else W_t[k][ci][co] (or, with GRAD,
// the layer's own W [K][cout][cin], read flipped and transposed).
template <bool IS_BF16>
int forward_typed(const Map& m, int ksize, int cin, int cout, const _Float16* feats,
                  const _Float16* wp, bool grad, const float* bias, _Float16* out,
                  hipStream_t stream) {
  const int path = kernel_path(m.n, m.active_pairs, cin, cout, ksize);
  if (path < 0) return path;
  if (path == 1 && staged_takes(m, ksize, cin, cout))
    return forward_staged(m, cin, cout, IS_BF16, feats, wp, bias, out, stream);
  if (path == 1) {
    switch (cin) {
      case 32: return dispatch_cout<32, IS_BF16>(m, ksize, feats, wp, bias, out, cout, stream);
      case 64: return dispatch_cout<64, IS_BF16>(m, ksize, feats, wp, bias, out, cout, stream);
      case 128: return dispatch_cout<128, IS_BF16>(m, ksize, feats, wp, bias, out, cout, stream);
      case 256: return dispatch_cout<256, IS_BF16>(m, ksize, feats, wp, bias, out, cout, stream);
      default: break;
    }
  }
  const int64_t items = m.n * cout;
  // a grid-stride loop over (row, column) items
  const unsigned blocks = static_cast<unsigned>(std::min<int64_t>((items + 255) / 256, 1 << 20));
  const int B = 256;
  auto go = [&](auto k3, auto gr) {
    constexpr bool K3 = decltype(k3)::value, GR = decltype(gr)::value;
    k_fwd_valu<K3, IS_BF16, GR><<<blocks, B, 0, stream>>>(K3 ? m.nbr : nullptr,
                                                          K3 ? m.order : nullptr, m.n, feats, wp,
                                                          bias, out, cin, cout);
  };
  using T = std::true_type;
  using F = std::false_type;
  if (ksize == 3)
    grad ? go(T{}, T{}) : go(T{}, F{});
  else
    grad ? go(F{}, T{}) : go(F{}, F{});
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

// Rearranges W [K][cin][cout] for a forward with cin_t x cout_t channels
// (W itself, or with grad the input gradient's W[K-1-k]^T: cin_t = cout,
// cout_t = cin) into wp.
int prepare_into(const _Float16* W, int K, int cin, int cout, bool grad, _Float16* wp,
                 hipStream_t stream) {
  const int cin_t = grad ? cout : cin, cout_t = grad ? cin : cout;
  const int64_t total = static_cast<int64_t>(K) * cin * cout;
  const int B = 256;
  if (use_mfma(cin_t, cout_t))
    k_prepare_mfma<<<static_cast<unsigned>((total / 8 + B - 1) / B), B, 0, stream>>>(
        W, K, cin_t, cout_t, grad, wp);
  else
    k_prepare_plain<<<static_cast<unsigned>((total + B - 1) / B), B, 0, stream>>>(
        W, K, cin_t, cout_t, grad, wp);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

// ---------------------------------------------------------------------------
// per-device staging of weights passed as they are
// ---------------------------------------------------------------------------

// The largest prepared MFMA layer: 27 taps x 256 x 1024 (or 1024 x 256 for an
// input gradient) 16-bit elements.
constexpr size_t kStageBytes = size_t{kTaps3} * 256 * 1024 * 2;

// Buffers per device: the first kStageSlots - 1 streams that forward on W
// each own one for good, so their forwards need no ordering against other
// streams; any further streams share the last, ordered by an event.
constexpr int kStageSlots = 4;
struct Stage {
  std::mutex mu;
  _Float16* ptr[kStageSlots] = {};            // this device's staging buffers
  hipStream_t owner[kStageSlots - 1] = {};    // the stream owning each private buffer
  int owned = 0;                              // private buffers taken (in order)
  hipEvent_t done = nullptr;     // shared buffer: recorded after the last forward that read it
  hipStream_t last = nullptr;    // the stream of that forward
  bool recorded = false;
};
constexpr int kMaxDevices = 64;
Stage g_stages[kMaxDevices];

// A forward with weights as the caller holds them: for the MFMA kernels they
// are rearranged into a staging buffer of the device first: the stream's own
// buffer (the stream's order alone protects it), or, past the first
// kStageSlots - 1 streams, the shared one. Forwards on different streams are
// ordered around the shared buffer by an event (the stream waits for the
// previous user's event, and records its own after its launches); while the
// stream is being captured into a graph no event is used.
template <bool IS_BF16>
int forward_raw(const Map& m, int ksize, int cin, int cout, const _Float16* feats,
                const _Float16* W, bool grad, const float* bias, _Float16* out,
                hipStream_t stream) {
  // cin, cout: the channels of this forward (an input gradient's are the
  // layer's swapped); W: the layer's weights
  const int path = kernel_path(m.n, m.active_pairs, cin, cout, ksize);
  if (path < 0) return path;
  if (path == 0)
    return forward_typed<IS_BF16>(m, ksize, cin, cout, feats, W, grad, bias, out, stream);
  const int K = ksize == 3 ? kTaps3 : 1;
  if (static_cast<size_t>(K) * cin * cout * 2 > kStageBytes)
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "internal: %d x %d weights exceed the stage",
                     cin, cout);
  Stage& sg = g_stages[m.device];
  std::lock_guard<std::mutex> lock(sg.mu);
  if (!sg.ptr[0] || !sg.done)  // a map build on the device sets both up
    return set_error(SUBMCONV_ERR_INVALID_ARG, "internal: no weight stage on device %d", m.device);
  // the stream's own buffer, a free one it takes, or the shared one
  int slot = kStageSlots - 1;
  for (int i = 0; i < sg.owned; ++i)
    if (sg.owner[i] == stream) slot = i;
  if (slot == kStageSlots - 1 && sg.owned < kStageSlots - 1) {
    slot = sg.owned++;
    sg.owner[slot] = stream;
  }
  _Float16* const buf = sg.ptr[slot];
  const bool shared = slot == kStageSlots - 1;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  bool capturing = false;
  if (shared) {
    capturing =
        hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone;
    (void)hipGetLastError();  // a failed query is not this call's error
    if (!capturing && sg.recorded && sg.last != stream)
      SUBMCONV_HIP_CHECK(hipStreamWaitEvent(stream, sg.done, 0));
  }
  // the layer's W is [K][cin][cout], or [K][cout][cin] for an input gradient
  const int st = prepare_into(W, K, grad ? cout : cin, grad ? cin : cout, grad, buf, stream);
  if (st != SUBMCONV_OK) return st;
  const int fs = forward_typed<IS_BF16>(m, ksize, cin, cout, feats, buf, false, bias, out,
                                        stream);
  if (shared && !capturing) {
    SUBMCONV_HIP_CHECK(hipEventRecord(sg.done, stream));
    sg.recorded = true;
    sg.last = stream;
  }
  return fs;
}

// Checks shared by every forward entry point; n == 0 is handled by the caller.
int check_call(const Map& m, const void* feats, const void* w, const void* out, const float* bias) {
  if (!feats || !w || !out) return set_error(SUBMCONV_ERR_INVALID_ARG, "feats, W or out is NULL");
  if ((reinterpret_cast<uintptr_t>(feats) | reinterpret_cast<uintptr_t>(w) |
       reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(bias)) & 15)
    return set_error(SUBMCONV_ERR_INVALID_ARG,
                     "feats, W, out and bias must be 16-byte aligned");
  int dev = -1;
  SUBMCONV_HIP_CHECK(hipGetDevice(&dev));
  if (dev != m.device)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "the map is on device %d, the current device is %d",
                     m.device, dev);
  if (m.device < 0 || m.device >= kMaxDevices)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "device %d out of range", m.device);
  return SUBMCONV_OK;
}

}  // namespace

// Sets up the device's weight stage (one allocation of kStageSlots buffers
// and one event per device, kept until the process ends); every map build
// calls it, so that a forward, which always has a map, finds it and
// allocates nothing.
int ensure_weight_stage(int device) {
  if (device < 0 || device >= kMaxDevices)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "device %d out of range", device);
  Stage& sg = g_stages[device];
  std::lock_guard<std::mutex> lock(sg.mu);
  if (!sg.ptr[0]) {
    void* p = nullptr;
    SUBMCONV_HIP_CHECK(hipMalloc(&p, kStageSlots * kStageBytes));
    for (int i = 0; i < kStageSlots; ++i)
      sg.ptr[i] = static_cast<_Float16*>(p) + i * (kStageBytes / 2);
  }
  // the event only orders forwards on other streams of this device behind
  // the buffer's last user (hipStreamWaitEvent), so it needs no system-scope
  // fence (its cache writeback and invalidation)
  if (!sg.done)
    SUBMCONV_HIP_CHECK(
        hipEventCreateWithFlags(&sg.done, hipEventDisableTiming | hipEventDisableSystemFence));
  return SUBMCONV_OK;
}

}  // namespace submconv

using namespace submconv;

extern "C" int submconv_forward_kernel(int64_t n, int64_t active_pairs, int32_t cin, int32_t cout,
                                       int32_t ksize) {
  clear_error();
  const int st = check_shape(ksize, cin, cout);
  if (st != SUBMCONV_OK) return st;
  if (n < 0 || active_pairs < 0)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "negative row or pair count");
  const int path = kernel_path(n, active_pairs, cin, cout, ksize);
  // a map built with default flags has a staged plan when it is dense
  if (path == 1 && ksize == 3 && staged_shape(cin, cout) && n > 0 &&
      active_pairs >= int64_t{kStageMinPairsPerRow} * n)
    return 2;
  return path;
}

extern "C" int submconv_weights_create(int32_t ksize, int32_t cin, int32_t cout, int32_t dtype,
                                       uint32_t flags, submconv_weights_t* out) {
  clear_error();
  if (!out) return set_error(SUBMCONV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  const int st = check_shape(ksize, cin, cout);
  if (st != SUBMCONV_OK) return st;
  if (dtype != SUBMCONV_DTYPE_F16 && dtype != SUBMCONV_DTYPE_BF16)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "dtype = %d is not fp16 (0) or bf16 (1)", dtype);
  if (flags & ~SUBMCONV_PREP_INPUT_GRAD)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "unknown preparation flags 0x%x", flags);
  Weights w;
  SUBMCONV_HIP_CHECK(hipGetDevice(&w.device));
  w.ksize = ksize;
  w.cin = cin;
  w.cout = cout;
  w.dtype = dtype;
  w.flags = flags;
  const size_t bytes = static_cast<size_t>(ksize == 3 ? kTaps3 : 1) * cin * cout * 2;
  SUBMCONV_HIP_CHECK(hipMalloc(&w.buf, bytes));
  *out = new submconv_weights_s{w};
  return SUBMCONV_OK;
}

extern "C" int submconv_weights_set(submconv_weights_t h, const uint16_t* W, hipStream_t stream) {
  clear_error();
  if (!h || !W) return set_error(SUBMCONV_ERR_INVALID_ARG, "weights or W is NULL");
  if (reinterpret_cast<uintptr_t>(W) & 15)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "W must be 16-byte aligned");
  const Weights& w = h->w;
  int dev = -1;
  SUBMCONV_HIP_CHECK(hipGetDevice(&dev));
  if (dev != w.device)
    return set_error(SUBMCONV_ERR_INVALID_ARG,
                     "the weights are on device %d, the current device is %d", w.device, dev);
  return prepare_into(reinterpret_cast<const _Float16*>(W), w.ksize == 3 ? kTaps3 : 1, w.cin,
                      w.cout, w.flags & SUBMCONV_PREP_INPUT_GRAD, w.buf, stream);
}

extern "C" int submconv_weights_free(submconv_weights_t h) {
  clear_error();
  if (!h) return SUBMCONV_OK;
  const hipError_t e = hipFree(h->w.buf);
  delete h;
  SUBMCONV_HIP_CHECK(e);
  return SUBMCONV_OK;
}

// One forward of cin -> cout channels on weights W (the layer's, grad for an
// input gradient) or on a prepared handle's buffer.
static int forward_entry(submconv_map_t map, const uint16_t* feats_u16, const uint16_t* W,
                         const float* bias, uint16_t* out_u16, int32_t cin, int32_t cout,
                         int32_t ksize, int32_t dtype, bool grad, bool prepared,
                         hipStream_t stream) {
  if (!map) return set_error(SUBMCONV_ERR_INVALID_ARG, "map is NULL");
  if (dtype != SUBMCONV_DTYPE_F16 && dtype != SUBMCONV_DTYPE_BF16)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "dtype = %d is not fp16 (0) or bf16 (1)", dtype);
  const int st = check_shape(ksize, cin, cout);
  if (st != SUBMCONV_OK) return st;
  const Map& m = map->m;
  if (m.n == 0) return SUBMCONV_OK;
  const int cs = check_call(m, feats_u16, W, out_u16, bias);
  if (cs != SUBMCONV_OK) return cs;
  const _Float16* feats = reinterpret_cast<const _Float16*>(feats_u16);
  const _Float16* w = reinterpret_cast<const _Float16*>(W);
  _Float16* out = reinterpret_cast<_Float16*>(out_u16);
  if (prepared) {
    if (dtype == SUBMCONV_DTYPE_BF16)
      return forward_typed<true>(m, ksize, cin, cout, feats, w, false, bias, out, stream);
    return forward_typed<false>(m, ksize, cin, cout, feats, w, false, bias, out, stream);
  }
  if (dtype == SUBMCONV_DTYPE_BF16)
    return forward_raw<true>(m, ksize, cin, cout, feats, w, grad, bias, out, stream);
  return forward_raw<false>(m, ksize, cin, cout, feats, w, grad, bias, out, stream);
}

extern "C" int submconv_forward_dtype(submconv_map_t map, const uint16_t* feats,
                                      const uint16_t* W, const float* bias, uint16_t* out,
                                      int32_t cin, int32_t cout, int32_t ksize, int32_t dtype,
                                      hipStream_t stream) {
  clear_error();
  return forward_entry(map, feats, W, bias, out, cin, cout, ksize, dtype, false, false, stream);
}

extern "C" int submconv_forward(submconv_map_t map, const uint16_t* feats, const uint16_t* W,
                                const float* bias, uint16_t* out, int32_t cin, int32_t cout,
                                int32_t ksize, hipStream_t stream) {
  clear_error();
  return forward_entry(map, feats, W, bias, out, cin, cout, ksize, SUBMCONV_DTYPE_F16, false,
                       false, stream);
}

extern "C" int submconv_forward_prepared(submconv_map_t map, const uint16_t* feats,
                                         submconv_weights_t h, const float* bias, uint16_t* out,
                                         hipStream_t stream) {
  clear_error();
  if (!h) return set_error(SUBMCONV_ERR_INVALID_ARG, "weights is NULL");
  const Weights& w = h->w;
  if (w.flags & SUBMCONV_PREP_INPUT_GRAD)
    return set_error(SUBMCONV_ERR_INVALID_ARG,
                     "these weights are prepared for the input gradient, not the forward");
  if (map && map->m.device != w.device)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "the map is on device %d, the weights on %d",
                     map->m.device, w.device);
  return forward_entry(map, feats, reinterpret_cast<const uint16_t*>(w.buf), bias, out, w.cin,
                       w.cout, w.ksize, w.dtype, false, true, stream);
}

extern "C" int submconv_backward_input_dtype(submconv_map_t map, const uint16_t* grad_out,
                                             const uint16_t* W, uint16_t* grad_in, int32_t cin,
                                             int32_t cout, int32_t ksize, int32_t dtype,
                                             hipStream_t stream) {
  clear_error();
  // the forward with the flipped, transposed kernel, cout -> cin channels
  return forward_entry(map, grad_out, W, nullptr, grad_in, cout, cin, ksize, dtype, true, false,
                       stream);
}

extern "C" int submconv_backward_input(submconv_map_t map, const uint16_t* grad_out,
                                       const uint16_t* W, uint16_t* grad_in, int32_t cin,
                                       int32_t cout, int32_t ksize, hipStream_t stream) {
  return submconv_backward_input_dtype(map, grad_out, W, grad_in, cin, cout, ksize,
                                       SUBMCONV_DTYPE_F16, stream);
}

extern "C" int submconv_backward_input_prepared(submconv_map_t map, const uint16_t* grad_out,
                                                submconv_weights_t h, uint16_t* grad_in,
                                                hipStream_t stream) {
  clear_error();
  if (!h) return set_error(SUBMCONV_ERR_INVALID_ARG, "weights is NULL");
  const Weights& w = h->w;
  if (!(w.flags & SUBMCONV_PREP_INPUT_GRAD))
    return set_error(SUBMCONV_ERR_INVALID_ARG,
                     "these weights are prepared for the forward, not the input gradient");
  if (map && map->m.device != w.device)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "the map is on device %d, the weights on %d",
                     map->m.device, w.device);
  return forward_entry(map, grad_out, reinterpret_cast<const uint16_t*>(w.buf), nullptr, grad_in,
                       w.cout, w.cin, w.ksize, w.dtype, false, true, stream);
}
