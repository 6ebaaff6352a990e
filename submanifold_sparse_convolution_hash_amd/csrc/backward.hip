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
#include <type_traits>
#include <utility>

#include "submconv_internal.h"

namespace submconv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kPairs = 32;          // pairs per group
constexpr int kRowPad = kPairs + 8; // LDS row (one channel): 32 pairs + 8 halves of padding
constexpr int kTargetBlocks = 1024; // workgroups to aim for (taps x tile runs)

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
    int32_t n_tiles, int32_t K, int32_t tpr, const _Float16* __restrict__ feats,
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
          const int64_t t_row = int64_t{t} * kTileRows + e.y;
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

struct Runs {
  int runs, tpr;
};
Runs runs_for(const Map& m, int K) {
  const int64_t nt = m.n_tiles;
  int64_t runs = (kTargetBlocks + K - 1) / K;
  if (runs > nt) runs = nt;
  if (runs < 1) runs = 1;
  const int64_t tpr = (nt + runs - 1) / runs;
  runs = (nt + tpr - 1) / tpr;
  return {static_cast<int>(runs), static_cast<int>(tpr)};
}

template <int CIN, int COUT>
int launch_w(const Map& m, int K, const _Float16* feats, const _Float16* grad_out, float* partial,
             float* dw, hipStream_t stream) {
  const Runs r = runs_for(m, K);
  k_bwd_weight<CIN, COUT><<<static_cast<unsigned>(r.runs * K), WCfg<CIN, COUT>::NT, 0, stream>>>(
      m.ent, m.tile_off, m.tile_cnt, m.order, m.n, static_cast<int32_t>(m.n_tiles), K, r.tpr,
      feats, grad_out, partial, static_cast<int32_t>(m.active_pairs));
  SUBMCONV_HIP_CHECK(hipGetLastError());
  const int64_t total = static_cast<int64_t>(K) * CIN * COUT;
  k_bwd_weight_reduce<<<static_cast<unsigned>((total + 255) / 256), 256, 0, stream>>>(
      partial, r.runs, K, CIN, COUT, dw);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

template <int CIN>
int dispatch_w(const Map& m, int K, int cout, const _Float16* feats, const _Float16* grad_out,
               float* partial, float* dw, hipStream_t stream) {
  switch (cout) {
    case 32: return launch_w<CIN, 32>(m, K, feats, grad_out, partial, dw, stream);
    case 64: return launch_w<CIN, 64>(m, K, feats, grad_out, partial, dw, stream);
    case 96: return launch_w<CIN, 96>(m, K, feats, grad_out, partial, dw, stream);
    case 128: return launch_w<CIN, 128>(m, K, feats, grad_out, partial, dw, stream);
    case 160: return launch_w<CIN, 160>(m, K, feats, grad_out, partial, dw, stream);
    case 192: return launch_w<CIN, 192>(m, K, feats, grad_out, partial, dw, stream);
    case 224: return launch_w<CIN, 224>(m, K, feats, grad_out, partial, dw, stream);
    case 256: return launch_w<CIN, 256>(m, K, feats, grad_out, partial, dw, stream);
    default: return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "internal: Cout = %d", cout);
  }
}

}  // namespace
}  // namespace submconv

using namespace submconv;

extern "C" int64_t submconv_backward_weight_workspace_bytes(submconv_map_t map, int32_t cin,
                                                            int32_t cout, int32_t ksize) {
  if (!map) return set_error(SUBMCONV_ERR_INVALID_ARG, "map is NULL");
  if (ksize != 1 && ksize != 3) return set_error(SUBMCONV_ERR_INVALID_ARG, "ksize = %d", ksize);
  if (cin <= 0 || cout <= 0 || cin % 8 || cout % 8 || cin > 1024 || cout > 1024)
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "Cin = %d, Cout = %d", cin, cout);
  if (!use_mfma_w(cin, cout) || map->m.n == 0) return 0;
  const int K = ksize == 3 ? kTaps3 : 1;
  const Runs r = runs_for(map->m, K);
  return static_cast<int64_t>(r.runs) * K * cin * cout * static_cast<int64_t>(sizeof(float));
}

extern "C" int submconv_backward_weight(submconv_map_t map, const uint16_t* feats,
                                        const uint16_t* grad_out, float* grad_w, void* workspace,
                                        int32_t cin, int32_t cout, int32_t ksize,
                                        hipStream_t stream) {
  clear_error();
  const int64_t ws = submconv_backward_weight_workspace_bytes(map, cin, cout, ksize);
  if (ws < 0) return static_cast<int>(ws);
  const Map& m = map->m;
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
  const _Float16* f = reinterpret_cast<const _Float16*>(feats);
  const _Float16* g = reinterpret_cast<const _Float16*>(grad_out);
  float* part = static_cast<float*>(workspace);
  if (ws > 0 && m.n * cin * 2 < (int64_t{1} << 31) - 64 && m.n * cout * 2 < (int64_t{1} << 31) - 64) {
    switch (cin) {
      case 32: return dispatch_w<32>(m, K, cout, f, g, part, grad_w, stream);
      case 64: return dispatch_w<64>(m, K, cout, f, g, part, grad_w, stream);
      case 96: return dispatch_w<96>(m, K, cout, f, g, part, grad_w, stream);
      case 128: return dispatch_w<128>(m, K, cout, f, g, part, grad_w, stream);
      case 160: return dispatch_w<160>(m, K, cout, f, g, part, grad_w, stream);
      case 192: return dispatch_w<192>(m, K, cout, f, g, part, grad_w, stream);
      case 224: return dispatch_w<224>(m, K, cout, f, g, part, grad_w, stream);
      case 256: return dispatch_w<256>(m, K, cout, f, g, part, grad_w, stream);
      default: break;
    }
  }
  const int64_t items = static_cast<int64_t>(K) * cin * (cout / 8);
  k_bwd_weight_valu<<<static_cast<unsigned>((items + 255) / 256), 256, 0, stream>>>(
      K == kTaps3 ? m.nbr : nullptr, m.order, m.n, K, f, g, cin, cout, grad_w);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
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
