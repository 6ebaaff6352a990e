// Staged SubMConv3d weight gradient for dense maps (32 or 64 channels), on
// gfx950.
//
// dW[k] = sum over the rows i with a neighbour j at tap k of feats[j]^T
// grad_out[i] (the gradient of the forward's per-tap products feats[j] @ W[k];
// the issue #1 thread lists a weight-gradient kernel next to the forward).
// On a dense map the pair-by-pair kernel gathers each feature row ~21 times;
// here the forward's staged plan is reused: a unit of up to 128 consecutive
// processing rows has its distinct neighbour rows (at most kStageCap) and its
// own output-gradient rows in LDS, and each tap's product over the unit's
// rows is one small GEMM whose K dimension is the unit's rows:
//   dW[k] += X_k^T dY, X_k[r] = the staged row of row r's neighbour at tap k
// (the zero row where it has none), dY[r] = grad_out at row r.
//
// Wave w owns taps k = w, w + 4, ... and keeps their dW in registers for all
// its units (v_mfma_f32_32x32x16: A = X_k^T, input channels x rows; B = dY,
// rows x output channels). Both operands are columns of row-major LDS rows,
// read with ds_read_b64_tr_b16, which transposes 16 lanes' 4-element row
// pieces into 4-element column pieces; the dY operand is read once per unit.
// One workgroup per CU walks its XCD's units; the next unit's staged rows,
// gradient rows and table are loaded into registers and written to the other
// LDS buffers while the current unit multiplies. Each workgroup writes its
// fp32 partial dW (all 27 taps) to the workspace, and a second kernel adds
// the partials in workgroup order: the result does not depend on scheduling.
#include "submconv_internal.h"

namespace submconv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ half8 bload_h8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// LDS-only barrier: loads in flight stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int CIN, int COUT>
struct CfgB {
  static constexpr int NT = 256;
  static constexpr int MB = CIN / 32, NB = COUT / 32;  // 32-channel blocks of dW
  static constexpr int RC = CIN / 8, YC = COUT / 8;    // 16-byte chunks of a row
  static constexpr int XB = (kStageCap + 1) * RC;      // staged rows and the zero row
  static constexpr int YB = kStageUnitRows * YC;       // the unit's gradient rows
  static constexpr int IW = kTaps3 * kStageUnitRows / 2;  // the table, in words
  static constexpr int IJ = (IW + NT - 1) / NT;           // its words per thread
  static constexpr int SQ = kStageCap * RC / NT;          // staged-row chunks per thread
  static constexpr int SPT = SQ / 4;                      // ... per tap, taps 2..5
  static constexpr int YQ = YB / NT;                      // gradient chunks per thread
  static constexpr int TPW = 7;                           // taps per wave (the last has 6)
  static_assert((CIN == 32 || CIN == 64) && (COUT == 32 || COUT == 64) && CIN * COUT < 64 * 64,
                "shape");
  static_assert(SQ % 4 == 0 && YB % NT == 0 && kStageCap * RC % NT == 0, "layout");
};

// chunk c of staged row s sits at s*RC + (c ^ swz(s)): rows that follow each
// other fill the 16 bank groups of a 256-byte line
template <int RC>
__host__ __device__ constexpr int swz(int s) {
  return (s / (16 / RC)) & (RC - 1);
}

template <int CIN, int COUT>
__global__ __launch_bounds__(256, 1) void k_bwd_weight_staged(
    const int4* __restrict__ units, int n_units, int per_xcd, int wpx,
    const int32_t* __restrict__ srows, const uint32_t* __restrict__ sidx2, int64_t istride2,
    const int32_t* __restrict__ order, int64_t n, const _Float16* __restrict__ feats,
    const _Float16* __restrict__ grad_out, float* __restrict__ partial) {
  using C = CfgB<CIN, COUT>;
  constexpr int MB = C::MB, NB = C::NB, RC = C::RC, YC = C::YC, SQ = C::SQ, SPT = C::SPT;
  __shared__ half8 xs[2][C::XB];  // staged feature rows, two buffers in turn
  __shared__ half8 ys[C::YB];     // the unit's gradient rows (zero past its rows)
  // per tap and lane pattern q8 (16 rows each, below), the swizzled chunk
  // base E*RC + swz(E) of each row's staged neighbour (the zero row's for
  // none), two buffers in turn
  __shared__ uint16_t ptab[2][kTaps3 * kStageUnitRows];

  const int bid = blockIdx.x;
  const int xcd = bid & 7, j0 = bid >> 3;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ntaps = (kTaps3 - w + 3) / 4;  // this wave's taps k = w + 4 i
  auto tap = [&](int i) { return w + 4 * i < kTaps3 ? w + 4 * i : kTaps3 - 1; };

  const __amdgpu_buffer_rsrc_t rf = make_rsrc(feats, static_cast<uint32_t>(n * CIN * 2));
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(grad_out, static_cast<uint32_t>(n * COUT * 2));

  // Transposed reads: lane (gq = lane / 16, sl = lane % 16) names row
  // 8 (gq / 2) + 4 r + sl / 4 of a 16-row K step and channels
  // 16 (gq % 2) + 4 (sl % 4) .. + 3 of a 32-channel block, and receives
  // channel 16 (gq % 2) + sl of rows 8 (gq / 2) + 4 r + 0..3; reads r = 0, 1
  // make the MFMA operand (lane: channel lane % 32, rows 8 (lane / 32) + 0..7).
  const int gq = lane >> 4, sl = lane & 15;
  const int c0 = 2 * (gq & 1) + ((sl & 3) >> 1);  // the lane's chunk in a 32-channel block
  const int piece = (sl & 1) * 4;                  // its 4-element piece in the chunk (halves)
  const int q8 = 4 * (gq >> 1) + (sl >> 2);        // its row pattern: rows 16 kk + 8 (q8/4) + 4 r + q8%4
  auto tr = [&](const half8* base, int chunk_base, int blk) {
    // chunk_base: row * rc + swizzle of that row; the lane's chunk of block blk
    const _Float16* hb = reinterpret_cast<const _Float16*>(base);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4s*)(hb + ((chunk_base ^ (c0 | (blk << 2))) << 3) + piece));
  };

  // staging: staged-row chunk slots tid + 256 q (row tid / RC + (256 / RC) q,
  // slot tid % RC, which holds chunk (tid % RC) ^ swz(row), the same for all q)
  const int cslot = (tid % RC) ^ swz<RC>(tid / RC);
  auto load_rows = [&](const int4& dd, int (&ROW)[SQ]) {
#pragma unroll
    for (int q = 0; q < SQ; ++q) {
      const int sr = tid / RC + (C::NT / RC) * q;
      ROW[q] = srows[dd.z + (sr < dd.w ? sr : dd.w - 1)];
    }
  };
  // gradient rows: slot tid + 256 z is unit row r = (tid + 256 z) / YC, slot
  // j = tid % YC, holding chunk j ^ (r % YC)
  auto load_grows = [&](const int4& dd, int (&GR)[C::YQ]) {
#pragma unroll
    for (int z = 0; z < C::YQ; ++z) {
      const int r = (tid + C::NT * z) / YC, rr = r < dd.y ? r : dd.y - 1;
      const int o = (order ? order : srows)[order ? dd.x + rr : dd.z];
      GR[z] = r < dd.y ? (order ? o : static_cast<int>(dd.x + rr)) : -1;
    }
  };
  auto load_gchunks = [&](const int (&GR)[C::YQ], half8 (&YG)[C::YQ]) {
#pragma unroll
    for (int z = 0; z < C::YQ; ++z) {
      const int r = (tid + C::NT * z) / YC, c = (tid % YC) ^ (r % YC);
      YG[z] = bload_h8(rg, GR[z] < 0 ? 0x80000000u
                                     : static_cast<uint32_t>(GR[z]) * (COUT * 2) + c * 16);
    }
  };
  auto load_itab = [&](const int4& dd, uint32_t (&IT)[C::IJ]) {
    const int pw = (dd.y + 1) >> 1;
#pragma unroll
    for (int i = 0; i < C::IJ; ++i) {
      const int e0 = tid + C::NT * i, e = e0 < C::IW ? e0 : C::IW - 1;
      const int k = e >> 6, pp = e & 63;
      IT[i] = sidx2[k * istride2 + (dd.x >> 1) + (pp < pw ? pp : pw - 1)];
    }
  };
  // table word e (tap k, rows r and r + 1) into the lane-pattern layout:
  // row r = 16 kk + 8 a + 4 b + c sits at k 128 + (4 a + c) 16 + 2 kk + b
  auto put_itab = [&](int buf, int rows, const uint32_t (&IT)[C::IJ]) {
    constexpr int zbase = kStageCap * RC;  // the zero row's chunk base (swz = 0)
    static_assert(swz<RC>(kStageCap) == 0, "zero row swizzle");
#pragma unroll
    for (int i = 0; i < C::IJ; ++i) {
      const int e0 = tid + C::NT * i, e = e0 < C::IW ? e0 : C::IW - 1;
      const int k = e >> 6;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int r = 2 * (e & 63) + hh;
        const int s = static_cast<int>((IT[i] >> (16 * hh)) & 0xFFFFu);
        const int v = r < rows && s != kStageNone ? s * RC + swz<RC>(s) : zbase;
        const int pos = k * kStageUnitRows + (4 * ((r >> 3) & 1) + (r & 3)) * 16 +
                        2 * (r >> 4) + ((r >> 2) & 1);
        ptab[buf][pos] = static_cast<uint16_t>(v);
      }
    }
  };

  float16v acc[C::TPW][MB][NB];
#pragma unroll
  for (int i = 0; i < C::TPW; ++i)
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[i][a][b] = float16v{};

  auto unit_of = [&](int ju) { return ju < per_xcd ? xcd * per_xcd + ju : n_units; };
  int ju = j0;
  int u = unit_of(ju);
  if (u < n_units) {
    int4 d = units[u];
    // ---- prologue: the first unit's rows, gradient rows, table; the zero rows ----
    int ROW[SQ];
    {
      load_rows(d, ROW);
      int GR[C::YQ];
      load_grows(d, GR);
      uint32_t IT[C::IJ];
      load_itab(d, IT);
      half8 G[SQ], YG[C::YQ];
#pragma unroll
      for (int q = 0; q < SQ; ++q)
        G[q] = bload_h8(rf, static_cast<uint32_t>(ROW[q]) * (CIN * 2) + cslot * 16);
      load_gchunks(GR, YG);
#pragma unroll
      for (int q = 0; q < SQ; ++q) xs[0][tid + C::NT * q] = G[q];
#pragma unroll
      for (int z = 0; z < C::YQ; ++z) ys[tid + C::NT * z] = YG[z];
      put_itab(0, d.y, IT);
      if (tid < 2 * RC) xs[tid / RC][kStageCap * RC + tid % RC] = half8{};
    }
    __syncthreads();

    int xb = 0;
    while (true) {
      const int ju_n = ju + wpx;
      const int u_n = unit_of(ju_n);
      const bool has_next = u_n < n_units;
      // (past the last unit the staging repeats this unit's, unused)
      const int4 d_n = has_next ? units[u_n] : d;
      const half8* cx = xs[xb];
      half8* nx = xs[xb ^ 1];
      const uint16_t* pt = ptab[xb];

      // ---- the unit's gradient operand, all K steps; then ys is free ----
      half8 BY[NB][8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int r0 = 16 * kk + 8 * (gq >> 1) + (sl >> 2), r1 = r0 + 4;
          const v4s lo = tr(ys, r0 * YC + (r0 % YC), b);
          const v4s hi = tr(ys, r1 * YC + (r1 % YC), b);
          BY[b][kk] = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
      auto load_p = [&](int k, uint32_t (&P)[8]) {
        const uint4* p4 = reinterpret_cast<const uint4*>(pt + k * kStageUnitRows + q8 * 16);
        const uint4 a = p4[0], b = p4[1];
        P[0] = a.x; P[1] = a.y; P[2] = a.z; P[3] = a.w;
        P[4] = b.x; P[5] = b.y; P[6] = b.z; P[7] = b.w;
      };
      uint32_t PE[2][8];
      load_p(tap(0), PE[0]);
      // A operands of half a tap (K steps 4 hh .. 4 hh + 3 of tap i), read a
      // half tap ahead of their MFMAs
      auto read_a = [&](const uint32_t (&P)[8], int hh, half8 (&A)[4][MB]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // rows 16 kk + 8 (q8/4) + 4 r + q8%4, r = 0, 1: entries 2 kk + r
          const uint32_t pw = P[4 * hh + q];
          const int p0 = static_cast<int>(pw & 0xFFFFu), p1 = static_cast<int>(pw >> 16);
#pragma unroll
          for (int a = 0; a < MB; ++a) {
            const v4s lo = tr(cx, p0, a), hi = tr(cx, p1, a);
            A[q][a] = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
        }
      };
      half8 AO[2][4][MB];
      read_a(PE[0], 0, AO[0]);
      lds_barrier();

      int GR[C::YQ];
      half8 YG[C::YQ];
      uint32_t IT[C::IJ];
      half8 G[2][SPT];
#pragma unroll
      for (int i = 0; i < C::TPW; ++i) {
        if (i == 0) {
          load_rows(d_n, ROW);
          load_grows(d_n, GR);
          load_itab(d_n, IT);
        }
        if (i == 1) load_gchunks(GR, YG);
        if (i >= 2 && i < 6) {
#pragma unroll
          for (int z = 0; z < SPT; ++z)
            G[i & 1][z] = bload_h8(rf, static_cast<uint32_t>(ROW[SPT * (i - 2) + z]) * (CIN * 2) +
                                           cslot * 16);
        }
        if (i + 1 < C::TPW) load_p(tap(i + 1), PE[(i + 1) & 1]);
        // (wave 3 also multiplies a seventh tap, tap 26 again, into an
        // accumulator it never writes out: no branch around the MFMAs)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int st = 2 * i + hh;
          if (hh == 0)
            read_a(PE[i & 1], 1, AO[(st + 1) & 1]);
          else if (i + 1 < C::TPW)
            read_a(PE[(i + 1) & 1], 0, AO[(st + 1) & 1]);
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int a = 0; a < MB; ++a)
#pragma unroll
              for (int b = 0; b < NB; ++b)
                acc[i][a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(AO[st & 1][q][a],
                                                                      BY[b][4 * hh + q],
                                                                      acc[i][a][b], 0, 0, 0);
          if constexpr (MB == 1 && NB == 1) {
            // 32 -> 32: each MFMA followed by two of the next half tap's
            // reads (left to the compiler, they sat right before their own
            // MFMA; measured 8 % slower; 64 -> 32 is not helped by this)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
              __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (i >= 3 && i < 7) {
#pragma unroll
          for (int z = 0; z < SPT; ++z) nx[tid + C::NT * (SPT * (i - 3) + z)] = G[(i - 1) & 1][z];
        }
        if (i == 3) {
#pragma unroll
          for (int z = 0; z < C::YQ; ++z) ys[tid + C::NT * z] = YG[z];
        }
        if (i == 4) put_itab(xb ^ 1, d_n.y, IT);
      }
      lds_barrier();  // the next unit is in place; this unit's buffers are free
      xb ^= 1;
      if (!has_next) break;
      ju = ju_n;
      d = d_n;
    }
  }

  // ---- this workgroup's partial dW of all 27 taps: D lane holds column
  // lane % 32 and rows 8 (j / 4) + 4 h + j % 4 (input channels) ----
  const int s32 = lane & 31, h = lane >> 5;
  float* pg = partial + static_cast<int64_t>(bid) * kTaps3 * CIN * COUT;
#pragma unroll
  for (int i = 0; i < C::TPW; ++i) {
    if (i < ntaps) {
      const int k = w + 4 * i;
#pragma unroll
      for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int ci = 32 * a + 8 * (j >> 2) + 4 * h + (j & 3), co = 32 * b + s32;
            pg[(static_cast<int64_t>(k) * CIN + ci) * COUT + co] = acc[i][a][b][j];
          }
    }
  }
}

// dW[e] = the sum of the blocks' partials of element e, block order: thread
// (s, f) adds blocks s, s + kStrands, ... of float4 f, then thread (0, f)
// adds the strands' sums in order.
constexpr int kStrands = 8;
__global__ __launch_bounds__(64 * kStrands) void k_bwd_weight_staged_reduce(
    const float4v* __restrict__ partial, int blocks, int64_t nf4, float4v* __restrict__ dw) {
  __shared__ float4v part[kStrands][64];
  const int f = threadIdx.x & 63, s = threadIdx.x >> 6;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 64 + f;
  float4v v = {0.f, 0.f, 0.f, 0.f};
  if (e < nf4)
    for (int b = s; b < blocks; b += kStrands) v += partial[static_cast<int64_t>(b) * nf4 + e];
  part[s][f] = v;
  __syncthreads();
  if (s == 0 && e < nf4) {
    float4v t = part[0][f];
#pragma unroll
    for (int q = 1; q < kStrands; ++q) t += part[q][f];
    dw[e] = t;
  }
}

template <int CIN, int COUT>
int per_cu() {
  static const int v = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &nb, reinterpret_cast<const void*>(k_bwd_weight_staged<CIN, COUT>), CfgB<CIN, COUT>::NT,
            0) != hipSuccess)
      nb = 1;
    return nb < 1 ? 1 : nb;
  }();
  return v;
}

// workgroups of the staged weight gradient on this map, 0 when it does not apply
template <int CIN, int COUT>
int64_t blocks_for(const Map& m) {
  int cus = 256;
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, m.device);
  const int64_t per_xcd = (m.staged.n_units + 7) / 8;
  const int64_t slots = int64_t{cus < 8 ? 1 : cus / 8} * per_cu<CIN, COUT>();
  return 8 * (per_xcd < slots ? per_xcd : slots);
}

template <int CIN, int COUT>
int launch(const Map& m, const _Float16* feats, const _Float16* grad_out, float* partial,
           float* dw, hipStream_t stream) {
  const Staged& S = m.staged;
  const int64_t per_xcd = (S.n_units + 7) / 8;
  const int64_t nb = blocks_for<CIN, COUT>(m);
  const int wpx = static_cast<int>(nb / 8);
  k_bwd_weight_staged<CIN, COUT><<<static_cast<unsigned>(nb), CfgB<CIN, COUT>::NT, 0, stream>>>(
      S.units, static_cast<int>(S.n_units), static_cast<int>(per_xcd), wpx, S.rows,
      reinterpret_cast<const uint32_t*>(S.idx), staged_idx_stride(m.n) / 2, m.order, m.n, feats,
      grad_out, partial);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  const int64_t nf4 = int64_t{kTaps3} * CIN * COUT / 4;
  k_bwd_weight_staged_reduce<<<static_cast<unsigned>((nf4 + 63) / 64), 64 * kStrands, 0, stream>>>(
      reinterpret_cast<const float4v*>(partial), static_cast<int>(nb), nf4,
      reinterpret_cast<float4v*>(dw));
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

}  // namespace

int64_t staged_wgrad_blocks(const Map& m, int ksize, int cin, int cout) {
  if (ksize != 3 || m.staged.n_units <= 0 || m.staged.n_units > (int64_t{1} << 28)) return 0;
  if (cin == 32 && cout == 32) return blocks_for<32, 32>(m);
  if (cin == 64 && cout == 32) return blocks_for<64, 32>(m);
  if (cin == 32 && cout == 64) return blocks_for<32, 64>(m);
  return 0;
}

int backward_weight_staged(const Map& m, int cin, int cout, const _Float16* feats,
                           const _Float16* grad_out, float* partial, float* dw,
                           hipStream_t stream) {
  if (cin == 32 && cout == 32) return launch<32, 32>(m, feats, grad_out, partial, dw, stream);
  if (cin == 64 && cout == 32) return launch<64, 32>(m, feats, grad_out, partial, dw, stream);
  if (cin == 32 && cout == 64) return launch<32, 64>(m, feats, grad_out, partial, dw, stream);
  return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "staged weight gradient: Cin %d, Cout %d", cin,
                   cout);
}

}  // namespace submconv
