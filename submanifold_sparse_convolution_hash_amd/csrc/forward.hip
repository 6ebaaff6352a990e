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

template <int CIN, int COUT_T, int NW>
struct Cfg {
  static constexpr int M = kTileRows;      // output rows per tile
  static constexpr int S = CIN / 32;       // 32-channel MFMA K steps
  static constexpr int CW = COUT_T / NW;   // output columns per wave
  static constexpr int NB = CW / 16;       // 16-column MFMA blocks per wave
  static constexpr int NQ = COUT_T / 4;    // float4 chunks per accumulator row
  static_assert(CIN % 32 == 0 && CIN <= 256, "CIN");
  static_assert(CW % 16 == 0 && NB >= 1, "COUT_T/NW");
  static_assert((NQ & (NQ - 1)) == 0, "NQ must be a power of two");
};

// One 16-row group of the tile's schedule (uniform across the wave).
struct Group {
  int p;      // processing position (0 = centre tap)
  int start;  // first entry of the group within the tile's list
  int cnt;    // live rows in the group (<= 16; <= 0 past the end)
};

// Group g of the schedule whose per-position entry counts, entry offsets and
// group offsets sit in lanes p = 0..26 (cnt_p, off_p, goff_p).
__device__ __forceinline__ Group group_at(int g, int cnt_p, int off_p, int goff_p, int lane) {
  const uint64_t m = __ballot(lane < kTaps3 && cnt_p > 0 && goff_p <= g);
  const int p = m ? 63 - __clzll(m) : 0;
  const int j = g - __builtin_amdgcn_readlane(goff_p, p);
  Group gr;
  gr.p = p;
  gr.start = __builtin_amdgcn_readlane(off_p, p) + 16 * j;
  const int left = __builtin_amdgcn_readlane(cnt_p, p) - 16 * j;
  gr.cnt = m ? (left < 16 ? left : 16) : 0;
  return gr;
}

template <int CIN, int COUT_T, int NW, bool K3, int PIPE>
__global__ __launch_bounds__(64 * NW) void k_fwd_mfma(
    const int2* __restrict__ ent, const int32_t* __restrict__ tile_off,
    const uint16_t* __restrict__ tile_cnt, const int32_t* __restrict__ order, int64_t n,
    const _Float16* __restrict__ feats, const _Float16* __restrict__ wp,
    const float* __restrict__ bias, _Float16* __restrict__ out, int cout, int n_tiles, int n_ct,
    int tiles_per_xcd) {
  using C = Cfg<CIN, COUT_T, NW>;
  constexpr int M = C::M;
  constexpr int NB = C::NB;
  constexpr int S = C::S;
  __shared__ float4v acc[M * C::NQ];

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

  // ---- schedule: entries per processing position, in lanes p < 27 ----
  int cnt_p = 0;
  int64_t ent0 = 0, ent1 = 0;
  if (K3) {
    if (lane < kTaps3) cnt_p = tile_cnt[static_cast<int64_t>(tile) * kTaps3 + lane];
    ent0 = tile_off[tile];
    ent1 = tile_off[tile + 1];
  } else {
    cnt_p = lane == 0 ? rows_here : 0;
  }
  const int ng_p = (cnt_p + 15) >> 4;
  const int off_p = excl_scan_wave(cnt_p, lane);
  const int goff_p = excl_scan_wave(ng_p, lane);
  const int n_groups = __builtin_amdgcn_readlane(goff_p + ng_p, kTaps3 - 1);

  const int s = lane & 15;   // slot (row of the group) this lane gathers
  const int kg = lane >> 4;  // channel quarter this lane covers
  const int cwb = c0 + w * C::CW;
  const int qw = (w * C::CW) >> 2;

  // bias of this lane's output columns, added once by the centre tap
  float4v bias4[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) bias4[cb][i] = bias ? bias[cwb + cb * 16 + 4 * kg + i] : 0.f;

  const __amdgpu_buffer_rsrc_t rf = make_rsrc(feats, static_cast<uint32_t>(n * CIN * 2));
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(wp, static_cast<uint32_t>((K3 ? kTaps3 : 1) * CIN * cout * 2));
  const __amdgpu_buffer_rsrc_t re = make_rsrc(ent + ent0, static_cast<uint32_t>((ent1 - ent0) * 8));

  auto sched = [&](int g) { return group_at(g, cnt_p, off_p, goff_p, lane); };
  auto tap_of = [&](const Group& gr) { return K3 ? tap_at(gr.p) : 0; };
  // entry {source row, row in tile} of this lane's slot in group gr
  auto load_entry = [&](const Group& gr) -> int2 {
    const bool live = s < gr.cnt;
    if (K3) return bload_i2(re, live ? static_cast<uint32_t>(gr.start + s) * 8u : kOob);
    int2 e;
    e.x = static_cast<int>(t0) + gr.start + s;
    e.y = gr.start + s;
    return e;
  };
  auto load_b = [&](int2 e, bool live, half8 (&B)[S]) {
    const uint32_t base = static_cast<uint32_t>(e.x) * (CIN * 2) + kg * (CIN / 2);
#pragma unroll
    for (int st = 0; st < S; ++st) B[st] = bload_h8(rf, live ? base + st * 16 : kOob);
  };
  auto load_a = [&](int tap, bool need, half8 (&A)[NB][S]) {
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      const uint32_t base =
          static_cast<uint32_t>(((tap * (cout / 16) + (cwb >> 4) + cb) * S) * 1024 + lane * 16);
#pragma unroll
      for (int st = 0; st < S; ++st)
        if (need) A[cb][st] = bload_h8(rw, base + st * 1024);
    }
  };

  // ---- software pipeline over the groups of the tile ----
  // Group g is multiplied in step g. Step g requests, in this order, the
  // weights of group g + LA (only if its tap changes: out-of-range loads
  // would still cost address-unit cycles), the feature rows of group g + LA
  // and the entry of
  // group g + U. Every buffer is a ring indexed by g mod U and the loop is
  // unrolled by U, so no register with a load in flight is ever copied, the
  // wait counts are static, and each load has LA steps to arrive.
  constexpr int U = PIPE;
  constexpr int LA = U / 2;
  half8 AL[U][NB][S];  // weights requested for a group (zeros if unchanged)
  bool needA[U];
  half8 Acur[NB][S];   // weights of the tap being multiplied
  half8 B[U][S];       // feature rows
  int2 E[U];           // entries {source row, row in tile}
  Group G[U];          // schedule

#pragma unroll
  for (int i = 0; i < U; ++i) {
    G[i] = sched(i);
    E[i] = load_entry(G[i]);
  }
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    needA[i] = i == 0 || tap_of(G[i]) != tap_of(G[i - 1]);
    load_a(tap_of(G[i]), needA[i], AL[i]);
    load_b(E[i], s < G[i].cnt, B[i]);
  }

  auto step = [&](int g, auto qc) {
    constexpr int q = decltype(qc)::value;  // g mod U
    constexpr int qn = (q + LA) % U;        // (g + LA) mod U
    const Group cur = G[q];
    const bool live = s < cur.cnt;
    const int r = E[q].y;
    // group g + LA: weights (if its tap changes) and feature rows
    const Group gn = sched(g + LA);
    const Group gp = sched(g + LA - 1);
    needA[qn] = tap_of(gn) != tap_of(gp);
    load_a(tap_of(gn), needA[qn], AL[qn]);
    load_b(E[qn], s < G[qn].cnt, B[qn]);
    // accumulator rows this lane will update (read before the multiply)
    float4v old[NB];
    if (live && cur.p != 0) {
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int qq = qw + cb * 4 + kg;
        old[cb] = acc[r * C::NQ + (qq ^ (r & (C::NQ - 1)))];
      }
    }
    // weights of group g
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
      for (int st = 0; st < S; ++st) Acur[cb][st] = needA[q] ? AL[q][cb][st] : Acur[cb][st];
    // group g: multiply and accumulate
    float4v d[NB];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      d[cb] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < S; ++st)
        d[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Acur[cb][st], B[q][st], d[cb], 0, 0, 0);
    }
    if (live) {
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int qq = qw + cb * 4 + kg;
        acc[r * C::NQ + (qq ^ (r & (C::NQ - 1)))] = cur.p == 0 ? d[cb] + bias4[cb] : old[cb] + d[cb];
      }
    }
    // group g + U: entry, into the slot group g has just released
    G[q] = sched(g + U);
    E[q] = load_entry(G[q]);
  };

  for (int g = 0; g < n_groups; g += U) {
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (step(g + I, std::integral_constant<int, I>{}), ...);
    }(std::make_integer_sequence<int, U>{});
  }
  __syncthreads();

  // ---- epilogue: fp32 -> fp16 (RNE), rows to their caller index ----
  constexpr int C8 = COUT_T / 8;
  for (int idx = tid; idx < rows_here * C8; idx += 64 * NW) {
    const int r = idx / C8;
    const int c8 = idx - r * C8;
    const int q0 = 2 * c8, q1 = 2 * c8 + 1;
    const float4v a = acc[r * C::NQ + (q0 ^ (r & (C::NQ - 1)))];
    const float4v b = acc[r * C::NQ + (q1 ^ (r & (C::NQ - 1)))];
    half8 h;
    h[0] = static_cast<_Float16>(a[0]);
    h[1] = static_cast<_Float16>(a[1]);
    h[2] = static_cast<_Float16>(a[2]);
    h[3] = static_cast<_Float16>(a[3]);
    h[4] = static_cast<_Float16>(b[0]);
    h[5] = static_cast<_Float16>(b[1]);
    h[6] = static_cast<_Float16>(b[2]);
    h[7] = static_cast<_Float16>(b[3]);
    const int64_t orow = (K3 && order) ? order[t0 + r] : t0 + r;
    *reinterpret_cast<half8*>(out + orow * cout + c0 + 8 * c8) = h;
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

// MFMA fragment order: for tap k, 16-column block cb, K step st and lane l,
// 8 consecutive fp16 values W[k][ci][co] with co = 16*cb + (l % 16) and
// ci = (l / 16) * (Cin / 4) + 8*st + j, j = 0..7: one contiguous 1 KiB run per
// (k, cb, st), loaded by a wave with one 16-byte load per lane.
__global__ void k_prepare_mfma(const _Float16* __restrict__ W, int K, int cin, int cout,
                               _Float16* __restrict__ wp) {
  const int64_t total = static_cast<int64_t>(K) * cin * cout;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int S = cin / 32;
  const int j = static_cast<int>(idx & 7);
  const int l = static_cast<int>((idx >> 3) & 63);
  int64_t rest = idx >> 9;
  const int st = static_cast<int>(rest % S);
  rest /= S;
  const int cb = static_cast<int>(rest % (cout / 16));
  const int k = static_cast<int>(rest / (cout / 16));
  const int co = 16 * cb + (l & 15);
  const int ci = (l >> 4) * (cin / 4) + 8 * st + j;
  wp[idx] = W[(static_cast<int64_t>(k) * cin + ci) * cout + co];
}

__global__ void k_copy_halves(const _Float16* __restrict__ W, int64_t total, _Float16* __restrict__ wp) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx < total) wp[idx] = W[idx];
}

bool use_mfma(int cin, int cout) {
  const bool cin_ok = cin == 32 || cin == 64 || cin == 128 || cin == 256;
  return cin_ok && cout % 16 == 0;
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

template <int CIN, int COUT_T, int NW>
int launch_mfma(const Map& m, int ksize, const _Float16* feats, const _Float16* wp,
                const float* bias, _Float16* out, int cout, hipStream_t stream) {
  const int64_t n_tiles64 = (m.n + kTileRows - 1) / kTileRows;
  if (n_tiles64 > (int64_t{1} << 28))
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "too many rows");
  const int n_tiles = static_cast<int>(n_tiles64);
  const int n_ct = cout / COUT_T;
  const int tiles_per_xcd = (n_tiles + 7) / 8;
  const int64_t blocks = int64_t{8} * tiles_per_xcd * n_ct;
  constexpr int PIPE = CIN <= 128 ? 4 : 2;  // ring depth (registers scale with CIN)
  if (ksize == 3)
    k_fwd_mfma<CIN, COUT_T, NW, true, PIPE><<<static_cast<unsigned>(blocks), 64 * NW, 0, stream>>>(
        m.ent, m.tile_off, m.tile_cnt, m.order, m.n, feats, wp, bias, out, cout, n_tiles, n_ct,
        tiles_per_xcd);
  else
    k_fwd_mfma<CIN, COUT_T, NW, false, PIPE><<<static_cast<unsigned>(blocks), 64 * NW, 0, stream>>>(
        nullptr, nullptr, nullptr, nullptr, m.n, feats, wp, bias, out, cout, n_tiles, n_ct,
        tiles_per_xcd);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

template <int CIN>
int dispatch_cout(const Map& m, int ksize, const _Float16* feats, const _Float16* wp,
                  const float* bias, _Float16* out, int cout, hipStream_t stream) {
  if (cout % 128 == 0) return launch_mfma<CIN, 128, 4>(m, ksize, feats, wp, bias, out, cout, stream);
  if (cout % 64 == 0) return launch_mfma<CIN, 64, 4>(m, ksize, feats, wp, bias, out, cout, stream);
  if (cout % 32 == 0) return launch_mfma<CIN, 32, 2>(m, ksize, feats, wp, bias, out, cout, stream);
  return launch_mfma<CIN, 16, 1>(m, ksize, feats, wp, bias, out, cout, stream);
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
