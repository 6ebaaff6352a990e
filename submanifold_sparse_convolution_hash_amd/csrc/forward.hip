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
// Design of the MFMA kernel (one workgroup = one tile of M output rows x
// COUT_T output columns; nothing is shared between workgroups, no atomics):
//   1. Prologue: the tile's 27 x M neighbour entries are read once; a wave
//      ballot per (tap, 64 rows) gives per-tap row masks, from which every
//      tap gets a compacted list of the tile rows that have that neighbour
//      (sentinel rows are dropped here, so no zero rows are ever multiplied
//      beyond the padding of the last 16-row group of a tap).
//   2. Main loop, per wave and without barriers: each wave owns COUT_T/NW
//      output columns and walks all 16-row groups (centre tap first, then
//      taps 0..26). For a group it gathers the 16 neighbour feature rows
//      straight from HBM/L2 into MFMA B fragments (contiguous 16-byte loads),
//      multiplies them with the tap's weight fragments on
//      v_mfma_f32_16x16x32_f16 (fp32 accumulate), and adds the 16x16 results
//      into an fp32 accumulator tile held in LDS. The centre tap initialises
//      the accumulator (with the bias), every later tap read-modify-writes it;
//      rows are unique within a tap and columns are private to a wave, so
//      there are no conflicts and the order of additions is fixed.
//   3. Epilogue: one rounding to fp16 (round to nearest even) and coalesced
//      row stores at the caller's row index.
#include "submconv_internal.h"

namespace submconv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kMaxChannels = 1024;

// Processing position p -> tap: the centre first (it initialises the
// accumulator), then the other 26 taps in ascending order.
__device__ __forceinline__ int tap_at(int p) { return p == 0 ? kCenterTap : (p <= kCenterTap ? p - 1 : p); }

__device__ __forceinline__ int excl_scan_wave(int v, int lane) {
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x - v;
}

// ---------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------

template <int CIN, int COUT_T, int M, int NW>
struct Cfg {
  static constexpr int S = CIN / 32;       // 32-channel MFMA K steps
  static constexpr int CW = COUT_T / NW;   // output columns per wave
  static constexpr int NB = CW / 16;       // 16-column MFMA blocks per wave
  static constexpr int CHUNKS = M / 64;    // 64-row ballot chunks per tile
  static constexpr int NQ = COUT_T / 4;    // float4 chunks per accumulator row
  static constexpr int MAXG = kTaps3 * M / 16;
  static_assert(CIN % 32 == 0 && CIN <= 256, "CIN");
  static_assert(CW % 16 == 0 && NB >= 1, "COUT_T/NW");
  static_assert(M % 64 == 0 && M <= 256, "M");
  static_assert((NQ & (NQ - 1)) == 0, "NQ must be a power of two");
};

template <int CIN, int COUT_T, int M, int NW>
__global__ __launch_bounds__(64 * NW) void k_fwd_mfma(
    const int32_t* __restrict__ nbr, const int32_t* __restrict__ order, int64_t n, int ksize,
    const _Float16* __restrict__ feats, const _Float16* __restrict__ wp,
    const float* __restrict__ bias, _Float16* __restrict__ out, int cout, int n_tiles, int n_ct,
    int tiles_per_xcd) {
  using C = Cfg<CIN, COUT_T, M, NW>;
  __shared__ float4v acc[M * C::NQ];
  __shared__ uint8_t lrow[kTaps3 * M];
  __shared__ uint64_t masks[kTaps3 * C::CHUNKS];
  __shared__ uint32_t gtab[C::MAXG];

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

  // ---- 1. per-tap row masks ----
  if (ksize == 3) {
    for (int ch = w; ch < C::CHUNKS; ch += NW) {
      const int r = ch * 64 + lane;
      const bool valid = r < rows_here;
      int32_t v[kTaps3];
#pragma unroll
      for (int k = 0; k < kTaps3; ++k) v[k] = valid ? nbr[static_cast<int64_t>(k) * n + t0 + r] : -1;
#pragma unroll
      for (int k = 0; k < kTaps3; ++k) {
        const uint64_t m = __ballot(v[k] >= 0);
        if (lane == 0) masks[k * C::CHUNKS + ch] = m;
      }
    }
  }
  __syncthreads();

  // per-position counts and offsets (every wave computes them; lanes p < 27)
  int cnt_p = 0;
  if (ksize == 3) {
    if (lane < kTaps3) {
      const int k = tap_at(lane);
#pragma unroll
      for (int ch = 0; ch < C::CHUNKS; ++ch) cnt_p += __popcll(masks[k * C::CHUNKS + ch]);
    }
  } else {
    cnt_p = lane == 0 ? rows_here : 0;
  }
  const int ng_p = (cnt_p + 15) >> 4;
  const int off_p = excl_scan_wave(cnt_p, lane);
  const int goff_p = excl_scan_wave(ng_p, lane);
  const int n_groups = __shfl(goff_p + ng_p, kTaps3 - 1, 64);

  // compacted row lists for the off-centre taps
  if (ksize == 3) {
    for (int ch = w; ch < C::CHUNKS; ch += NW) {
      const int r = ch * 64 + lane;
      const uint64_t below = (1ull << lane) - 1ull;
      for (int p = 1; p < kTaps3; ++p) {
        const int k = tap_at(p);
        int base = __shfl(off_p, p, 64);
        for (int c2 = 0; c2 < ch; ++c2) base += __popcll(masks[k * C::CHUNKS + c2]);
        const uint64_t m = masks[k * C::CHUNKS + ch];
        if ((m >> lane) & 1ull) lrow[base + __popcll(m & below)] = static_cast<uint8_t>(r);
      }
    }
  }
  if (w == 0 && lane < kTaps3) {
    for (int j = 0; j < ng_p; ++j) {
      const int left = cnt_p - 16 * j;
      gtab[goff_p + j] = static_cast<uint32_t>(off_p + 16 * j) |
                         (static_cast<uint32_t>(left < 16 ? left : 16) << 16) |
                         (static_cast<uint32_t>(lane) << 24);
    }
  }
  __syncthreads();

  // ---- 2. main loop: groups of 16 compacted rows ----
  const int s = lane & 15;
  const int kg = lane >> 4;
  const int cwb = c0 + w * C::CW;  // first output column of this wave
  const int qw = (w * C::CW) >> 2; // first float4 chunk of this wave in the tile
  half8 A[C::NB][C::S];
  int kcur = -1;
  const half8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int g = 0; g < n_groups; ++g) {
    const uint32_t e = gtab[g];
    const int start = static_cast<int>(e & 0xffffu);
    const int cnt = static_cast<int>((e >> 16) & 0xffu);
    const int p = static_cast<int>(e >> 24);
    const bool valid = s < cnt;
    const int kw = ksize == 3 ? tap_at(p) : 0;
    int r = 0;
    int64_t src = 0;
    if (valid) {
      if (p == 0) {
        r = start + s;
        src = (ksize == 3 && order) ? order[t0 + r] : t0 + r;
      } else {
        r = lrow[start + s];
        src = nbr[static_cast<int64_t>(kw) * n + t0 + r];
      }
    }
    half8 B[C::S];
    const _Float16* fp = feats + src * CIN + kg * (CIN / 4);
#pragma unroll
    for (int st = 0; st < C::S; ++st)
      B[st] = valid ? *reinterpret_cast<const half8*>(fp + 8 * st) : zero8;
    if (kw != kcur) {
      kcur = kw;
#pragma unroll
      for (int cb = 0; cb < C::NB; ++cb) {
        const _Float16* wq =
            wp + ((static_cast<int64_t>(kw) * (cout / 16) + (cwb >> 4) + cb) * C::S) * 512 + lane * 8;
#pragma unroll
        for (int st = 0; st < C::S; ++st) A[cb][st] = *reinterpret_cast<const half8*>(wq + st * 512);
      }
    }
#pragma unroll
    for (int cb = 0; cb < C::NB; ++cb) {
      float4v d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < C::S; ++st) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[cb][st], B[st], d, 0, 0, 0);
      if (valid) {
        const int q = qw + cb * 4 + kg;
        float4v* dst = &acc[r * C::NQ + (q ^ (r & (C::NQ - 1)))];
        if (p == 0) {
          if (bias) {
            const float* bp = bias + cwb + cb * 16 + 4 * kg;
            d[0] += bp[0];
            d[1] += bp[1];
            d[2] += bp[2];
            d[3] += bp[3];
          }
          *dst = d;
        } else {
          *dst += d;
        }
      }
    }
  }
  __syncthreads();

  // ---- 3. epilogue: fp32 -> fp16 (RNE), rows to their caller index ----
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
    const int64_t orow = (ksize == 3 && order) ? order[t0 + r] : t0 + r;
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

int check_shape(int32_t ksize, int32_t cin, int32_t cout) {
  if (ksize != 1 && ksize != 3)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "ksize = %d is not 1 or 3", ksize);
  if (cin <= 0 || cout <= 0 || cin % 8 || cout % 8 || cin > kMaxChannels || cout > kMaxChannels)
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE,
                     "Cin = %d, Cout = %d: both must be positive multiples of 8 up to %d", cin,
                     cout, kMaxChannels);
  return SUBMCONV_OK;
}

template <int CIN, int COUT_T, int M, int NW>
int launch_mfma(const Map& m, int ksize, const _Float16* feats, const _Float16* wp,
                const float* bias, _Float16* out, int cout, hipStream_t stream) {
  const int64_t n_tiles64 = (m.n + M - 1) / M;
  if (n_tiles64 > (int64_t{1} << 28))
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "too many rows");
  const int n_tiles = static_cast<int>(n_tiles64);
  const int n_ct = cout / COUT_T;
  const int tiles_per_xcd = (n_tiles + 7) / 8;
  const int64_t blocks = int64_t{8} * tiles_per_xcd * n_ct;
  k_fwd_mfma<CIN, COUT_T, M, NW><<<static_cast<unsigned>(blocks), 64 * NW, 0, stream>>>(
      ksize == 3 ? m.nbr : nullptr, ksize == 3 ? m.order : nullptr, m.n, ksize, feats, wp, bias,
      out, cout, n_tiles, n_ct, tiles_per_xcd);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

template <int CIN>
int dispatch_cout(const Map& m, int ksize, const _Float16* feats, const _Float16* wp,
                  const float* bias, _Float16* out, int cout, hipStream_t stream) {
  if (cout % 128 == 0)
    return launch_mfma<CIN, 128, 256, 4>(m, ksize, feats, wp, bias, out, cout, stream);
  if (cout % 64 == 0)
    return launch_mfma<CIN, 64, 256, 4>(m, ksize, feats, wp, bias, out, cout, stream);
  if (cout % 32 == 0)
    return launch_mfma<CIN, 32, 256, 2>(m, ksize, feats, wp, bias, out, cout, stream);
  return launch_mfma<CIN, 16, 256, 1>(m, ksize, feats, wp, bias, out, cout, stream);
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
  if (use_mfma(cin, cout)) {
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
