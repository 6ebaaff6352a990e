// SubMConv3d forward on gfx950: a fused, output-stationary gather-GEMM.
//
// out[i] = bias + sum_k feats[nbr[k][i]] @ W[k] is the fused-tap product
// [N, K^3*Cin] x [K^3*Cin, Cout] of the trellis_sparse_mlx README
// ("Performance": one matmul over all taps instead of 2*K^3 dispatches, and a
// cached gather index). The accumulator stays fp32 and the tile operands are
// fp16 (the mixed-precision shape of the "Fixed" list of the trellis-mac
// issue #1 thread); the absent-neighbour skip generalises that thread's
// skip-empty-V vote to single rows.
//
// Design of the MFMA kernel (one workgroup = one tile of 256 output rows x
// COUT_T output columns; nothing is shared between workgroups, no atomics):
//   * The map holds, per tile, the neighbours of every tap compacted into a
//     list of {neighbour row, row in tile} (built once with the map), so
//     absent neighbours cost nothing here: only the padding of the last
//     16-row group of a tap is multiplied by zeros.
//   * Each wave owns COUT_T/NW output columns and walks all 16-row groups of
//     the tile (centre tap first, then taps 0..26, in list order). For a group
//     it gathers the 16 feature rows straight into MFMA B fragments
//     (contiguous 16-byte loads per lane), multiplies them with the tap's
//     weight fragments on v_mfma_f32_16x16x32_f16 (fp32 accumulate) and adds
//     the 16x16 results into an fp32 accumulator tile in LDS. The centre tap
//     initialises the accumulator with the bias, later taps read-modify-write
//     it; rows are unique within a tap and columns are private to a wave, so
//     there are no conflicts and the order of additions is fixed.
//   * The group loop is software-pipelined: list entries are fetched PIPE
//     groups ahead, feature rows and weight fragments (when the tap
//     changes) PIPE/2 groups ahead.
//     Feature rows and entries go through buffer loads whose masked lanes
//     use an out-of-range offset (zeros, no memory traffic) instead of
//     branches; weight fragments are loaded only when the tap changes.
//   * Epilogue: one rounding to fp16 (round to nearest even) and coalesced
//     row stores at the caller's row index.
#include <type_traits>
#include <utility>

#include "submconv_internal.h"

namespace submconv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kMaxChannels = 1024;

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
__device__ __forceinline__ int2 bload_i2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(int2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// ---------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------

typedef float float16v __attribute__((ext_vector_type(16)));

template <int CIN, int COUT_T, bool K3, int NG, int NS>
struct Cfg {
  static constexpr int M = kTileRows;        // output rows per tile
  static constexpr int GR = 32;              // rows per group (MFMA 32x32x16)
  static constexpr int NW = COUT_T / 32;     // waves; each owns 32 output columns
  static constexpr int NT = 64 * NW;         // threads
  static constexpr int KS = CIN / 16;        // 16-channel MFMA K steps
  static constexpr int NQ = COUT_T / 4;      // float4 chunks per accumulator row
  static constexpr int RC = CIN / 8;         // 16-byte chunks per feature row
  static constexpr int GCH = GR * RC;        // chunks per group
  static constexpr int CPT = GCH >= NT ? GCH / NT : 1;  // chunks per loading thread
  static constexpr int NLOAD = GCH >= NT ? NT : GCH;    // loading threads
  static constexpr int NCG = M / GR;         // groups of the centre tap
  static constexpr int R = 2 * NG > 8 ? 2 * NG : 8;     // unroll factor
  // NS group tiles in LDS. With 4, a group's rows are stored two steps
  // before it is multiplied and read into registers one step before; with
  // 2, stored one step before and read in its own step.
  static constexpr int SD = NS == 4 ? 2 : 1;
  static constexpr int LB = SD + 2;          // chunks requested LB steps ahead
  static constexpr int LE = 2;               // entries LE steps before that
  static constexpr int LR = 3;               // rows of a group requested LR steps ahead
  static constexpr int RQ = 4;               // ring size of entries, chunks and rows
  static_assert(CIN % 32 == 0 && CIN <= 256, "CIN");
  static_assert(COUT_T % 32 == 0 && COUT_T <= 128, "COUT_T");
  static_assert(NS == 2 || NS == 4, "NS");
  static_assert(GCH % NT == 0 || NT % GCH == 0, "chunk split");
  static_assert((R / NG) % 2 == 0 && R % RQ == 0, "schedule");
  static_assert(LB - SD + 1 <= RQ && LE + 1 <= RQ && LR + 1 <= RQ, "ring");
};

template <int CIN, int COUT_T, bool K3, int NG, int NS>
__global__ __launch_bounds__(2 * COUT_T) void k_fwd_mfma(
    const int2* __restrict__ ent, const int32_t* __restrict__ tile_off,
    const uint16_t* __restrict__ tile_cnt, const int32_t* __restrict__ order, int64_t n,
    const _Float16* __restrict__ feats, const _Float16* __restrict__ wp,
    const float* __restrict__ bias, _Float16* __restrict__ out, int cout, int n_tiles, int n_ct,
    int tiles_per_xcd) {
  using C = Cfg<CIN, COUT_T, K3, NG, NS>;
  static_assert(C::NT == 2 * COUT_T, "launch bounds");
  constexpr int M = C::M, GR = C::GR, KS = C::KS, RC = C::RC, R = C::R;
  constexpr int SD = C::SD, LB = C::LB, LE = C::LE, LR = C::LR, RQ = C::RQ;
  constexpr int CPT = C::CPT, NCG = C::NCG;
  __shared__ float4v acc[M * C::NQ];
  __shared__ half8 bt[NS][C::GCH];  // feature rows of a group, 16-byte chunks, swizzled

  // Workgroups are dealt to the 8 XCDs round robin; give each XCD a
  // contiguous run of row tiles (and all column tiles of a row tile) so that
  // neighbouring tiles, which gather the same feature rows, share an L2.
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int li = bid >> 3;
  const int tl = li / n_ct;
  const int ct = li - tl * n_ct;
  const int tile = xcd * tiles_per_xcd + tl;
  if (tl >= tiles_per_xcd || tile >= n_tiles) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(tile) * M;
  const int rows_here = static_cast<int>(n - t0 < M ? n - t0 : M);
  const int c0 = ct * COUT_T;

  // ---- schedule: entries per processing position p, in lanes p < 27 ----
  int cnt_p = 0;
  int64_t ent0 = 0, ent1 = 0;
  if (K3) {
    if (lane < kTaps3) cnt_p = tile_cnt[static_cast<int64_t>(tile) * kTaps3 + lane];
    ent0 = tile_off[tile];
    ent1 = tile_off[tile + 1];
  } else {
    cnt_p = lane == 0 ? rows_here : 0;
  }
  const int off_p = excl_scan_wave(cnt_p, lane);
  // Static schedule: step f < NCG is group f of the centre tap (position 0);
  // step f >= NCG is group (f-NCG) % NG of position 1 + (f-NCG) / NG. Groups
  // beyond NG of a position are handled after the main loop.
  auto pos_of = [&](int f) { return f < NCG ? 0 : 1 + (f - NCG) / NG; };
  auto grp_of = [&](int f) { return f < NCG ? f : (f - NCG) % NG; };
  auto start_of = [&](int p, int j) {
    return __builtin_amdgcn_readlane(off_p, p < kTaps3 ? p : 0) + GR * j;
  };
  auto count_of = [&](int p, int j) {
    if (p >= (K3 ? kTaps3 : 1)) return 0;
    const int c = __builtin_amdgcn_readlane(cnt_p, p) - GR * j;
    return c < GR ? c : GR;
  };

  const __amdgpu_buffer_rsrc_t rf = make_rsrc(feats, static_cast<uint32_t>(n * CIN * 2));
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(wp, static_cast<uint32_t>((K3 ? kTaps3 : 1) * CIN * cout * 2));
  const __amdgpu_buffer_rsrc_t re = make_rsrc(ent + ent0, static_cast<uint32_t>((ent1 - ent0) * 8));

  // ---- loader role: this thread moves CPT 16-byte chunks of every group ----
  const bool loader = tid < C::NLOAD;
  int lrow[CPT], lpos[CPT];
  uint32_t lcol[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + C::NT * i;
    lrow[i] = c / RC;
    const int lc = c % RC;
    lcol[i] = static_cast<uint32_t>(lc * 16);
    lpos[i] = lrow[i] * RC + (lc ^ (lrow[i] & (RC - 1)));
  }
  auto entries_at = [&](int st, int cnt, int2 (&E)[CPT]) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const bool live = loader && lrow[i] < cnt;
      if (K3) {
        E[i] = bload_i2(re, live ? static_cast<uint32_t>(st + lrow[i]) * 8u : kOob);
        if (!live) E[i].y = -1;
      } else {
        E[i].x = static_cast<int>(t0) + st + lrow[i];
        E[i].y = live ? st + lrow[i] : -1;
      }
    }
  };
  auto load_entries = [&](int f, int2 (&E)[CPT]) {
    const int p = pos_of(f), j = grp_of(f);
    entries_at(start_of(p, j), count_of(p, j), E);
  };
  auto load_chunks = [&](const int2 (&E)[CPT], half8 (&D)[CPT]) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      D[i] = bload_h8(rf, E[i].y >= 0 ? static_cast<uint32_t>(E[i].x) * (CIN * 2) + lcol[i] : kOob);
  };
  auto store_chunks = [&](int slot, const half8 (&D)[CPT]) {
    if (loader) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) bt[slot][lpos[i]] = D[i];
    }
  };
  // row in tile of this lane's slot of the group of step f (-1: none)
  auto row_at = [&](int st, int cnt) -> int {
    const int sl = lane & 31;
    if (K3) {
      const int2 e = bload_i2(re, sl < cnt ? static_cast<uint32_t>(st + sl) * 8u : kOob);
      return sl < cnt ? e.y : -1;
    }
    return sl < cnt ? st + sl : -1;
  };
  auto load_row = [&](int f) -> int {
    const int p = pos_of(f), j = grp_of(f);
    return row_at(start_of(p, j), count_of(p, j));
  };

  // ---- MFMA role: this wave owns 32 output columns ----
  // v_mfma_f32_32x32x16_f16 computes out^T for the group: A = weights (lane:
  // column lane%32, channels (lane/32)*Cin/2 + 8*st + 0..7), B = gathered
  // rows (lane: slot lane%32, same channels), D: lane holds slot lane%32 and
  // columns 8*a + 4*(lane/32) + b in register 4*a + b.
  const int s32 = lane & 31;
  const int h = lane >> 5;
  const int cwb = c0 + w * 32;
  const int qw = w * 8;
  // weights of `tap` for this wave's 32 columns (one 16-byte load per K step)
  auto load_a = [&](int tap, half8 (&A)[KS]) {
    const uint32_t base =
        static_cast<uint32_t>(((tap * (cout / 32) + (cwb >> 5)) * KS) * 1024 + lane * 16);
#pragma unroll
    for (int st = 0; st < KS; ++st) A[st] = bload_h8(rw, base + st * 1024);
  };
  // LDS offsets (in chunks) of this lane's B fragments within a group tile
  int boff[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    const int lc = h * (CIN / 16) + st;
    boff[st] = s32 * RC + (lc ^ (s32 & (RC - 1)));
  }
  auto read_b = [&](int slot, half8 (&B)[KS]) {
#pragma unroll
    for (int st = 0; st < KS; ++st) B[st] = bt[slot][boff[st]];
  };
  // Multiply one group and add it to the accumulator rows of its slots. The
  // old values are read before the multiply and added after it, so the LDS
  // latency overlaps the MFMA chain. Lanes without a row read row 0 and
  // discard the result.
  auto multiply = [&](int r, bool centre, const half8 (&A)[KS], const half8 (&B)[KS]) {
    const bool live = r >= 0;
    const int rb = (r < 0 ? 0 : r) * C::NQ;
    const int rx = r & (C::NQ - 1);
    float4v old[4];
    if (!centre) {
#pragma unroll
      for (int a = 0; a < 4; ++a) old[a] = acc[rb + ((qw + 2 * a + h) ^ rx)];
    }
    float16v d = {};
#pragma unroll
    for (int st = 0; st < KS; ++st)
      d = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[st], B[st], d, 0, 0, 0);
    if (live) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float4v v = {d[4 * a], d[4 * a + 1], d[4 * a + 2], d[4 * a + 3]};
        acc[rb + ((qw + 2 * a + h) ^ rx)] = centre ? v : old[a] + v;
      }
    }
  };
  // LDS writes of this wave are complete, then all waves meet (an LDS-only
  // fence: outstanding global prefetches stay in flight across the barrier)
  auto lds_barrier = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  // ---- software pipeline over the static schedule ----
  // Step f: (NS = 4) read the B fragments of group f+1 from LDS into
  // registers; store the chunks of group f+SD (requested LB-SD steps
  // earlier); request the chunks of group f+LB, the rows of group f+LR and
  // the entries of group f+LB+LE; at the first group of a tap request the
  // weights of the next tap; multiply group f; barrier. Register rings are
  // indexed by f mod RQ and the loops are unrolled by R, so every load has a
  // static wait count; weights alternate between two register sets by tap
  // parity, B fragments by step parity.
  int2 E[RQ][CPT];
  half8 D[RQ][CPT];
  int RW[RQ];
  half8 AW[2][KS];
  half8 BF[2][KS];
#pragma unroll
  for (int f = 0; f < LB; ++f) load_entries(f, E[f % RQ]);
#pragma unroll
  for (int f = 0; f < LB; ++f) load_chunks(E[f % RQ], D[f % RQ]);
#pragma unroll
  for (int f = 0; f < LR; ++f) RW[f % RQ] = load_row(f);
#pragma unroll
  for (int f = LB; f < LB + LE; ++f) load_entries(f, E[f % RQ]);
  load_a(K3 ? kCenterTap : 0, AW[0]);
  if (K3) load_a(tap_at(1), AW[1]);
#pragma unroll
  for (int f = 0; f < SD; ++f) store_chunks(f, D[f % RQ]);
  lds_barrier();
  if (NS == 4) read_b(0, BF[0]);

  // ri: f mod R; ap: register set of the tap of step f; ts: first group of a tap
  auto step = [&](int f, auto ric, auto apc, auto tsc, bool centre) {
    constexpr int ri = decltype(ric)::value;
    constexpr int ap = decltype(apc)::value;
    constexpr bool ts = decltype(tsc)::value;
    if (ts) {
      const int pn = pos_of(f) + 1;  // past the last tap: reload it (harmless)
      load_a(tap_at(pn < kTaps3 ? pn : kTaps3 - 1), AW[1 - ap]);
    }
    if (NS == 4)
      read_b((ri + 1) % NS, BF[(ri + 1) & 1]);
    else
      read_b(ri & 1, BF[ri & 1]);
    store_chunks((ri + SD) % NS, D[(ri + SD) % RQ]);
    load_chunks(E[(ri + LB) % RQ], D[(ri + LB) % RQ]);
    const int r = RW[ri % RQ];
    RW[(ri + LR) % RQ] = load_row(f + LR);
    load_entries(f + LB + LE, E[(ri + LB + LE) % RQ]);
    multiply(r, centre, AW[ap], BF[ri & 1]);
    lds_barrier();
  };
  static_assert(NCG == 8 && NCG % RQ == 0, "centre steps");
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (step(I, std::integral_constant<int, I>{}, std::integral_constant<int, 0>{},
          std::false_type{}, true), ...);
  }(std::make_integer_sequence<int, NCG>{});
  if (K3) {
    for (int f = NCG; f < NCG + 26 * NG; f += R) {
      [&]<int... I>(std::integer_sequence<int, I...>) {
        (step(f + I, std::integral_constant<int, (NCG + I) % R>{},
              std::integral_constant<int, (1 + I / NG) % 2>{},
              std::integral_constant<bool, I % NG == 0>{}, false), ...);
      }(std::make_integer_sequence<int, R>{});
    }
    // groups beyond NG of a tap: one at a time, without pipelining
    for (int p = 1; p < kTaps3; ++p) {
      const int ngp = (__builtin_amdgcn_readlane(cnt_p, p) + GR - 1) / GR;
      if (ngp <= NG) continue;
      half8 A[KS];
      load_a(tap_at(p), A);
      for (int j = NG; j < ngp; ++j) {
        int2 e1[CPT];
        half8 d1[CPT], b1[KS];
        const int st = start_of(p, j), cnt = count_of(p, j);
        entries_at(st, cnt, e1);
        load_chunks(e1, d1);
        const int r1 = row_at(st, cnt);
        store_chunks(0, d1);
        lds_barrier();
        read_b(0, b1);
        multiply(r1, false, A, b1);
        lds_barrier();
      }
    }
  }
  __syncthreads();

  // ---- epilogue: fp32 -> fp16 (RNE), rows to their caller index ----
  constexpr int C8 = COUT_T / 8;
  for (int idx = tid; idx < rows_here * C8; idx += C::NT) {
    const int r = idx / C8;
    const int c8 = idx - r * C8;
    const int q0 = 2 * c8, q1 = 2 * c8 + 1;
    const float4v a = acc[r * C::NQ + (q0 ^ (r & (C::NQ - 1)))];
    const float4v b = acc[r * C::NQ + (q1 ^ (r & (C::NQ - 1)))];
    // the bias is added here, once, in fp32 before the single rounding
    float4v b0 = {0.f, 0.f, 0.f, 0.f}, b1 = {0.f, 0.f, 0.f, 0.f};
    if (bias) {
      b0 = *reinterpret_cast<const float4v*>(bias + c0 + 8 * c8);
      b1 = *reinterpret_cast<const float4v*>(bias + c0 + 8 * c8 + 4);
    }
    half8 hv;
    hv[0] = static_cast<_Float16>(a[0] + b0[0]);
    hv[1] = static_cast<_Float16>(a[1] + b0[1]);
    hv[2] = static_cast<_Float16>(a[2] + b0[2]);
    hv[3] = static_cast<_Float16>(a[3] + b0[3]);
    hv[4] = static_cast<_Float16>(b[0] + b1[0]);
    hv[5] = static_cast<_Float16>(b[1] + b1[1]);
    hv[6] = static_cast<_Float16>(b[2] + b1[2]);
    hv[7] = static_cast<_Float16>(b[3] + b1[3]);
    const int64_t orow = (K3 && order) ? order[t0 + r] : t0 + r;
    *reinterpret_cast<half8*>(out + orow * cout + c0 + 8 * c8) = hv;
  }
}

// ---------------------------------------------------------------------------
// VALU kernel for channel counts the MFMA tiles do not cover (multiples of 8)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_fwd_valu(
    const int32_t* __restrict__ nbr, const int32_t* __restrict__ order, int64_t n, int ksize,
    const _Float16* __restrict__ feats, const _Float16* __restrict__ w,
    const float* __restrict__ bias, _Float16* __restrict__ out, int cin, int cout) {
  const int c8n = cout / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n * c8n) return;
  const int64_t t = idx / c8n;
  const int o8 = static_cast<int>(idx - t * c8n);
  float a[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) a[q] = bias ? bias[o8 * 8 + q] : 0.f;
  const int K = ksize == 3 ? kTaps3 : 1;
  for (int k = 0; k < K; ++k) {
    int64_t j;
    if (ksize == 3) {
      j = nbr[static_cast<int64_t>(k) * n + t];
      if (j < 0) continue;
    } else {
      j = t;
    }
    const _Float16* f = feats + j * cin;
    const _Float16* wk = w + static_cast<int64_t>(k) * cin * cout + o8 * 8;
    for (int c = 0; c < cin; ++c) {
      const float fc = static_cast<float>(f[c]);
      const half8 wv = *reinterpret_cast<const half8*>(wk + static_cast<int64_t>(c) * cout);
#pragma unroll
      for (int q = 0; q < 8; ++q) a[q] += fc * static_cast<float>(wv[q]);
    }
  }
  half8 h;
#pragma unroll
  for (int q = 0; q < 8; ++q) h[q] = static_cast<_Float16>(a[q]);
  const int64_t orow = (ksize == 3 && order) ? order[t] : t;
  *reinterpret_cast<half8*>(out + orow * cout + o8 * 8) = h;
}

// ---------------------------------------------------------------------------
// weight preparation
// ---------------------------------------------------------------------------

// MFMA fragment order (v_mfma_f32_32x32x16_f16, weights as the A operand):
// for tap k, 32-column block cb, 16-channel K step st and lane l, 8
// consecutive fp16 values W[k][ci][co] with co = 32*cb + (l % 32) and
// ci = (l / 32) * (Cin / 2) + 8*st + j, j = 0..7: one contiguous 1 KiB run per
// (k, cb, st), loaded by a wave with one 16-byte load per lane.
__global__ void k_prepare_mfma(const _Float16* __restrict__ W, int K, int cin, int cout,
                               _Float16* __restrict__ wp) {
  const int64_t total = static_cast<int64_t>(K) * cin * cout;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int KS = cin / 16;
  const int j = static_cast<int>(idx & 7);
  const int l = static_cast<int>((idx >> 3) & 63);
  int64_t rest = idx >> 9;
  const int st = static_cast<int>(rest % KS);
  rest /= KS;
  const int cb = static_cast<int>(rest % (cout / 32));
  const int k = static_cast<int>(rest / (cout / 32));
  const int co = 32 * cb + (l & 31);
  const int ci = (l >> 5) * (cin / 2) + 8 * st + j;
  wp[idx] = W[(static_cast<int64_t>(k) * cin + ci) * cout + co];
}

__global__ void k_copy_halves(const _Float16* __restrict__ W, int64_t total, _Float16* __restrict__ wp) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx < total) wp[idx] = W[idx];
}

bool use_mfma(int cin, int cout) {
  if (cin == 256) return cout % 128 == 0;
  return (cin == 32 || cin == 64 || cin == 128) && cout % 32 == 0;
}

// The MFMA kernel addresses features, weights and lists through 32-bit
// buffer offsets below 2 GiB.
bool fits_buffers(const Map& m, int cin) {
  return m.n * cin * 2 < (int64_t{1} << 31) - 64 && m.active_pairs * 8 < (int64_t{1} << 31) - 64;
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

// 32-row groups per off-centre tap in the static schedule: the NG that
// minimises padded steps plus (about three times costlier) overflow groups,
// from the map's histogram of 16-row groups per (tile, off-centre tap).
int choose_ng(const Map& m) {
  const int cands[4] = {1, 2, 4, 8};
  int best = 8;
  double best_cost = 1e300;
  for (int ng : cands) {
    double over = 0;
    for (int b = 0; b < kNgHistBins; ++b) {
      const int ng32 = (b + 1) / 2;
      if (ng32 > ng) over += static_cast<double>(ng32 - ng) * m.ng_hist[b];
    }
    const double cost = static_cast<double>(m.n_tiles) * (8 + 26 * ng) + 3.0 * over;
    if (cost < best_cost) {
      best_cost = cost;
      best = ng;
    }
  }
  return best;
}

template <int CIN, int COUT_T, bool K3, int NG>
int launch_one(const Map& m, const _Float16* feats, const _Float16* wp, const float* bias,
               _Float16* out, int cout, hipStream_t stream) {
  // four group tiles when the LDS has room next to the accumulator
  constexpr int NS = 2;
  using Cf = Cfg<CIN, COUT_T, K3, NG, NS>;
  const int64_t n_tiles64 = (m.n + kTileRows - 1) / kTileRows;
  if (n_tiles64 > (int64_t{1} << 28))
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "too many rows");
  const int n_tiles = static_cast<int>(n_tiles64);
  const int n_ct = cout / COUT_T;
  const int tiles_per_xcd = (n_tiles + 7) / 8;
  const int64_t blocks = int64_t{8} * tiles_per_xcd * n_ct;
  k_fwd_mfma<CIN, COUT_T, K3, NG, NS><<<static_cast<unsigned>(blocks), Cf::NT, 0, stream>>>(
      K3 ? m.ent : nullptr, K3 ? m.tile_off : nullptr, K3 ? m.tile_cnt : nullptr,
      K3 ? m.order : nullptr, m.n, feats, wp, bias, out, cout, n_tiles, n_ct, tiles_per_xcd);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

template <int CIN, int COUT_T>
int launch_mfma(const Map& m, int ksize, const _Float16* feats, const _Float16* wp,
                const float* bias, _Float16* out, int cout, hipStream_t stream) {
  if (ksize == 1) return launch_one<CIN, COUT_T, false, 1>(m, feats, wp, bias, out, cout, stream);
  switch (choose_ng(m)) {
    case 1: return launch_one<CIN, COUT_T, true, 1>(m, feats, wp, bias, out, cout, stream);
    case 2: return launch_one<CIN, COUT_T, true, 2>(m, feats, wp, bias, out, cout, stream);
    case 4: return launch_one<CIN, COUT_T, true, 4>(m, feats, wp, bias, out, cout, stream);
    default: return launch_one<CIN, COUT_T, true, 8>(m, feats, wp, bias, out, cout, stream);
  }
}

template <int CIN>
int dispatch_cout(const Map& m, int ksize, const _Float16* feats, const _Float16* wp,
                  const float* bias, _Float16* out, int cout, hipStream_t stream) {
  // The LDS holds a 256 x COUT_T fp32 accumulator plus two 32-row groups of
  // Cin channels (at Cin = 256 and 128 columns that is exactly 160 KiB).
  if (cout % 128 == 0) return launch_mfma<CIN, 128>(m, ksize, feats, wp, bias, out, cout, stream);
  if constexpr (CIN <= 128) {
    if (cout % 64 == 0) return launch_mfma<CIN, 64>(m, ksize, feats, wp, bias, out, cout, stream);
    return launch_mfma<CIN, 32>(m, ksize, feats, wp, bias, out, cout, stream);
  }
  return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "internal: no MFMA tile for Cin = %d", CIN);
}

}  // namespace
}  // namespace submconv

using namespace submconv;

extern "C" int64_t submconv_prepared_weights_elems(int32_t ksize, int32_t cin, int32_t cout) {
  const int st = check_shape(ksize, cin, cout);
  if (st != SUBMCONV_OK) return st;
  return static_cast<int64_t>(ksize == 3 ? kTaps3 : 1) * cin * cout;
}

extern "C" int submconv_prepare_weights(const uint16_t* W, int32_t ksize, int32_t cin,
                                        int32_t cout, uint16_t* Wp, hipStream_t stream) {
  clear_error();
  const int st = check_shape(ksize, cin, cout);
  if (st != SUBMCONV_OK) return st;
  if (!W || !Wp) return set_error(SUBMCONV_ERR_INVALID_ARG, "W or Wp is NULL");
  const int K = ksize == 3 ? kTaps3 : 1;
  const int64_t total = static_cast<int64_t>(K) * cin * cout;
  const int B = 256;
  const unsigned grid = static_cast<unsigned>((total + B - 1) / B);
  const _Float16* w = reinterpret_cast<const _Float16*>(W);
  _Float16* p = reinterpret_cast<_Float16*>(Wp);
  if (use_mfma(cin, cout))
    k_prepare_mfma<<<grid, B, 0, stream>>>(w, K, cin, cout, p);
  else
    k_copy_halves<<<grid, B, 0, stream>>>(w, total, p);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

extern "C" int submconv_forward(submconv_map_t map, const uint16_t* feats_u16, const uint16_t* Wp,
                                const float* bias, uint16_t* out_u16, int32_t cin, int32_t cout,
                                int32_t ksize, hipStream_t stream) {
  clear_error();
  if (!map) return set_error(SUBMCONV_ERR_INVALID_ARG, "map is NULL");
  const int st = check_shape(ksize, cin, cout);
  if (st != SUBMCONV_OK) return st;
  const Map& m = map->m;
  if (m.n == 0) return SUBMCONV_OK;
  if (!feats_u16 || !Wp || !out_u16)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "feats, Wp or out is NULL");
  if ((reinterpret_cast<uintptr_t>(feats_u16) | reinterpret_cast<uintptr_t>(Wp) |
       reinterpret_cast<uintptr_t>(out_u16)) & 15)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "feats, Wp and out must be 16-byte aligned");
  const _Float16* feats = reinterpret_cast<const _Float16*>(feats_u16);
  const _Float16* wp = reinterpret_cast<const _Float16*>(Wp);
  _Float16* out = reinterpret_cast<_Float16*>(out_u16);
  if (use_mfma(cin, cout) && fits_buffers(m, cin)) {
    switch (cin) {
      case 32: return dispatch_cout<32>(m, ksize, feats, wp, bias, out, cout, stream);
      case 64: return dispatch_cout<64>(m, ksize, feats, wp, bias, out, cout, stream);
      case 128: return dispatch_cout<128>(m, ksize, feats, wp, bias, out, cout, stream);
      case 256: return dispatch_cout<256>(m, ksize, feats, wp, bias, out, cout, stream);
      default: break;
    }
  }
  const int64_t items = m.n * (cout / 8);
  const int B = 256;
  k_fwd_valu<<<static_cast<unsigned>((items + B - 1) / B), B, 0, stream>>>(
      ksize == 3 ? m.nbr : nullptr, ksize == 3 ? m.order : nullptr, m.n, ksize, feats, wp, bias,
      out, cin, cout);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}
