// Staged SubMConv3d forward with 256 output channels (128 or 256 input
// channels) for dense maps, on gfx950.
//
// The plan is the one the narrow staged forward uses (units of up to 128
// consecutive processing rows whose distinct neighbour rows, at most
// kStageCap, are staged once in LDS; a [27][128] table of where each row's
// neighbour sits among them; a zero row for absent neighbours). What differs
// is the width: at 256 channels a staged row is 512 bytes and a tap's weights
// 128 KiB, so
//  - one workgroup of 4 waves per CU, and wave w owns output columns
//    64 w .. 64 w + 63 of all the unit's rows (4 row blocks x 2 column blocks
//    of v_mfma_f32_32x32x16 accumulators, 128 fp32 registers per lane) and
//    multiplies all 27 taps itself: a row's sum runs over (slice, tap, K step)
//    in one fixed order, whatever the unit, and no partial sums are exchanged;
//  - the staged rows pass through LDS in 64-channel slices (128 bytes of
//    each staged row): two slice buffers in turn, the next slice (of this
//    unit, or the next unit's first) loaded into registers two chunks per
//    thread and tap while the current one is multiplied, and written to the
//    other buffer a tap later;
//  - each B fragment read from LDS feeds two MFMAs (both column blocks); a
//    tap's fragments are read a whole tap ahead (the address of each comes
//    from the LDS table, read two taps ahead), and its weights are loaded
//    once per unit and wave, a tap ahead.
// This is the fused [N, 27 Cin] x [27 Cin, Cout] product over a unit's rows
// (trellis_sparse_mlx README, "Performance"), with the gathered operand read
// from LDS instead of from memory for every (row, tap) pair.
#include "submconv_internal.h"

namespace submconv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));

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

// LDS-only barrier: the weight and staging loads in flight stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int CIN, int COUT>
struct CfgW {
  static constexpr int NT = 256;
  static constexpr int NSL = CIN / 64;   // slices per staged row
  static constexpr int KS = CIN / 16;    // MFMA K steps of a whole row (4 per slice)
  static constexpr int NCB = COUT / 32;  // 32-column blocks of the prepared weights
  static constexpr int SC = 8;           // 16-byte chunks of a row's slice
  static constexpr int BUF = (kStageCap + 1) * SC;  // one slice buffer, with the zero row
  static constexpr int IW = kTaps3 * kStageUnitRows / 2;  // the staged-row table, in words
  static constexpr int IJ = (IW + NT - 1) / NT;           // its words per thread
  static constexpr int SQ = kStageCap * SC / NT;          // a slice's chunks per thread
  static constexpr int T_ST = 2;   // taps T_ST .. T_ST + SQ / 2 - 1 load two chunks each
  static constexpr int T_NX = 12;  // the tap that requests rows, table and output rows
  static constexpr int T_IT = 20;  // the tap that writes the next unit's table
  static_assert((CIN == 128 || CIN == 256) && COUT == 256, "shape");
  static_assert(T_ST + SQ / 2 < T_NX && T_NX < T_IT && T_IT < kTaps3, "schedule");
  static_assert(kStageCap * SC % NT == 0 && SQ % 2 == 0, "layout");
};

// Persistent: the workgroups of XCD x (blockIdx % 8) walk that XCD's
// contiguous run of units (neighbouring units stage many of the same rows
// and share its L2), each taking every wpx-th unit of the run.
template <int CIN, int COUT, bool IS_BF16>
__global__ __launch_bounds__(256, 1) void k_fwd_staged_wide(
    const int4* __restrict__ units, int n_units, int per_xcd, int wpx,
    const int32_t* __restrict__ srows, const uint32_t* __restrict__ sidx2, int64_t istride2,
    const int32_t* __restrict__ order, int64_t n, const _Float16* __restrict__ feats,
    const _Float16* __restrict__ wp, const float* __restrict__ bias, _Float16* __restrict__ out) {
  using C = CfgW<CIN, COUT>;
  constexpr int NSL = C::NSL, KS = C::KS, NCB = C::NCB, SC = C::SC, SQ = C::SQ;
  __shared__ half8 stg[2][C::BUF];
  // staged rows of the unit's rows, [27][32][4]: tap k, row 32 rb + i at
  // k 128 + 4 i + rb, so that a lane reads its four row blocks' entries at once
  __shared__ uint32_t itab[2][C::IW];

  const int bid = blockIdx.x;
  const int xcd = bid & 7, j0 = bid >> 3;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int s32 = lane & 31, h = lane >> 5;

  const __amdgpu_buffer_rsrc_t rf = make_rsrc(feats, static_cast<uint32_t>(n * CIN * 2));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wp, static_cast<uint32_t>(kTaps3 * CIN * COUT * 2));
  // v_mfma_f32_32x32x16: A = weights (lane: column lane % 32 of the block;
  // K step st of lane half h: channels h CIN/2 + 8 st + 0..7), B = staged
  // rows (lane: row lane % 32 of the block, the same channels); D: lane holds
  // row lane % 32 and columns 8 a + 4 h + b in register 4 a + b. Slice p is
  // K steps 4 p .. 4 p + 3.
  auto load_a = [&](int k, int p, half8 (&A)[2][4]) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const uint32_t base =
          static_cast<uint32_t>(((k * NCB + 2 * w + cb) * KS + 4 * p) * 1024 + lane * 16);
#pragma unroll
      for (int st = 0; st < 4; ++st) A[cb][st] = bload_h8(rw, base + st * 1024);
    }
  };

  // Staging: thread tid moves slot j = tid % 8 of staged rows tid / 8 + 32 q
  // (q < SQ), the 16 bytes at LDS slot tid + 256 q of a slice buffer. Chunk c
  // of staged row s sits in slot c ^ swz(s), swz(s) = (s / 2) % 8, so that
  // the 16 lanes of a read pass that take consecutive staged rows hit
  // distinct banks; for this thread's rows swz is (tid / 16) % 8 for every q,
  // so its slot always holds the same chunk c of the slice: chunks 0..3 and
  // 4..7 are K steps 0..3 of lane halves 0 and 1.
  const int cslot = (tid & 7) ^ ((tid >> 4) & 7);
  const uint32_t cbyte = static_cast<uint32_t>(((cslot >> 2) * (CIN / 2) + 8 * (cslot & 3)) * 2);
  auto chunk_off = [&](int row, int p) {
    return static_cast<uint32_t>(row) * (CIN * 2) + cbyte + static_cast<uint32_t>(64 * p);
  };
  // the caller rows of unit dd's staged rows this thread moves (slots past
  // the unit's staged rows repeat its last one, and are never read)
  auto load_rows = [&](const int4& dd, int (&ROW)[SQ]) {
#pragma unroll
    for (int q = 0; q < SQ; ++q) {
      const int sr = (tid >> 3) + 32 * q;
      ROW[q] = srows[dd.z + (sr < dd.w ? sr : dd.w - 1)];
    }
  };
  // table words of unit dd (word e: tap e / 64, rows 2 (e % 64) and + 1;
  // units start on even rows and the table's stride is even; words past the
  // unit's rows repeat its last word)
  auto load_itab = [&](const int4& dd, uint32_t (&IT)[C::IJ]) {
    const int pw = (dd.y + 1) >> 1;
#pragma unroll
    for (int i = 0; i < C::IJ; ++i) {
      const int e0 = tid + C::NT * i, e = e0 < C::IW ? e0 : C::IW - 1;
      const int k = e >> 6, pp = e & 63;
      IT[i] = sidx2[k * istride2 + (dd.x >> 1) + (pp < pw ? pp : pw - 1)];
    }
  };
  auto put_itab = [&](int b, const uint32_t (&IT)[C::IJ]) {
    uint16_t* t16 = reinterpret_cast<uint16_t*>(itab[b]);
#pragma unroll
    for (int i = 0; i < C::IJ; ++i) {
      const int e0 = tid + C::NT * i, e = e0 < C::IW ? e0 : C::IW - 1;
      const int k = e >> 6, r = 2 * (e & 63);
      t16[k * kStageUnitRows + 4 * (r & 31) + (r >> 5)] = static_cast<uint16_t>(IT[i]);
      t16[k * kStageUnitRows + 4 * ((r + 1) & 31) + (r >> 5)] = static_cast<uint16_t>(IT[i] >> 16);
    }
  };

  auto unit_of = [&](int ju) { return ju < per_xcd ? xcd * per_xcd + ju : n_units; };
  int ju = j0;
  int u = unit_of(ju);
  if (u >= n_units) return;
  int4 d = units[u];

  // ---- prologue: the first unit's table and first slice, both zero rows ----
  int ROW[SQ];
  load_rows(d, ROW);
  {
    uint32_t IT[C::IJ];
    load_itab(d, IT);
    half8 G[SQ];
#pragma unroll
    for (int q = 0; q < SQ; ++q) G[q] = bload_h8(rf, chunk_off(ROW[q], 0));
#pragma unroll
    for (int q = 0; q < SQ; ++q) stg[0][tid + C::NT * q] = G[q];
    put_itab(0, IT);
    if (tid < 2 * SC) stg[tid / SC][kStageCap * SC + tid % SC] = half8{};
  }
  half8 An[2][4];  // the first tap's weights of the next slice
  load_a(0, 0, An);
  __syncthreads();

  float16v acc[4][2];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) acc[rb][0] = acc[rb][1] = float16v{};
  int sb = 0, ib = 0;
  while (true) {
    const int ju_n = ju + wpx;
    const int u_n = unit_of(ju_n);
    const bool has_next = u_n < n_units;
    // (past the last unit, the staging repeats this unit's rows, unused)
    const int4 d_n = has_next ? units[u_n] : d;
    const int rows = d.y;
    const int64_t t0 = d.x;
    const uint16_t* it16 = reinterpret_cast<const uint16_t*>(itab[ib]);
    int ORD[4];

    for (int p = 0; p < NSL; ++p) {
      const int pn = p + 1 < NSL ? p + 1 : 0;  // the slice staged meanwhile
      const half8* cur = stg[sb];
      half8* nxt = stg[sb ^ 1];
      // the staged row of this lane's row in each block at tap k (the zero
      // row where it has no neighbour, or past the unit's rows)
      auto load_e = [&](int k, int (&E)[4]) {
        const uint2 v = *reinterpret_cast<const uint2*>(it16 + k * kStageUnitRows + 4 * s32);
        const uint32_t e4[4] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16};
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          E[rb] = 32 * rb + s32 < rows && e4[rb] != kStageNone ? static_cast<int>(e4[rb]) : kStageCap;
      };
      auto load_b = [&](int e, half8 (&B)[4]) {
        const int sw = (e >> 1) & 7;
#pragma unroll
        for (int st = 0; st < 4; ++st) B[st] = cur[e * SC + ((4 * h + st) ^ sw)];
      };
      half8 A[2][2][4];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int st = 0; st < 4; ++st) A[0][cb][st] = An[cb][st];
      int E[3][4];  // table entries, two taps ahead
      half8 BB[2][4][4];  // staged-row fragments of two taps in turn
      load_e(0, E[0]);
      load_e(1, E[1]);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) load_b(E[0][rb], BB[0][rb]);
      half8 G[2][2];
      uint32_t IT[C::IJ];

#pragma unroll
      for (int t = 0; t < kTaps3; ++t) {
        if (t == C::T_NX) {
          // from the second-to-last slice on, the later staging reads the
          // next unit's rows; the next unit's table; this unit's output rows
          load_rows(p + 2 >= NSL ? d_n : d, ROW);
          load_itab(d_n, IT);
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            const int r = 32 * rb + s32, rr = r < rows ? r : rows - 1;
            const int o = (order ? order : srows)[order ? t0 + rr : d.z];
            ORD[rb] = order ? o : static_cast<int>(t0 + rr);
          }
        }
        if (t >= C::T_ST && t < C::T_ST + SQ / 2) {
          const int q0 = 2 * (t - C::T_ST);
          G[t & 1][0] = bload_h8(rf, chunk_off(ROW[q0], pn));
          G[t & 1][1] = bload_h8(rf, chunk_off(ROW[q0 + 1], pn));
        }
        if (t + 1 < kTaps3) load_a(t + 1, p, A[(t + 1) & 1]);
        else load_a(0, pn, An);
        if (t + 2 < kTaps3) load_e(t + 2, E[(t + 2) % 3]);
        // the next tap's fragments of all four row blocks are read before
        // this tap's MFMAs (a whole tap ahead); the MFMAs go two row blocks
        // at a time (the second pair only when the unit has more than 64
        // rows), both column blocks per B fragment
        if (t + 1 < kTaps3) {
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) load_b(E[(t + 1) % 3][rb], BB[(t + 1) & 1][rb]);
        }
#pragma unroll
        for (int rp = 0; rp < 4; rp += 2) {
          if (rp == 0 || rows > 64) {
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
              for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                  if constexpr (IS_BF16)
                    acc[rp + q][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, A[t & 1][cb][st]),
                        __builtin_bit_cast(bf16x8, BB[t & 1][rp + q][st]), acc[rp + q][cb], 0, 0, 0);
                  else
                    acc[rp + q][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        A[t & 1][cb][st], BB[t & 1][rp + q][st], acc[rp + q][cb], 0, 0, 0);
                }
          }
        }
        if (t > C::T_ST && t <= C::T_ST + SQ / 2) {
          const int q0 = 2 * (t - 1 - C::T_ST);
          nxt[tid + C::NT * q0] = G[(t - 1) & 1][0];
          nxt[tid + C::NT * (q0 + 1)] = G[(t - 1) & 1][1];
        }
        if (t == C::T_IT) put_itab(ib ^ 1, IT);
      }

      if (p + 1 == NSL) {
        // ---- epilogue: bias, one rounding, 8-byte pieces of the rows ----
        float4v b4[2][4];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int a = 0; a < 4; ++a)
            b4[cb][a] = bias ? *reinterpret_cast<const float4v*>(bias + 64 * w + 32 * cb + 8 * a + 4 * h)
                             : float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const bool live = 32 * rb + s32 < rows;
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
              const float16v& v = acc[rb][cb];
              const half4 o = {round16<IS_BF16>(v[4 * a] + b4[cb][a][0]),
                               round16<IS_BF16>(v[4 * a + 1] + b4[cb][a][1]),
                               round16<IS_BF16>(v[4 * a + 2] + b4[cb][a][2]),
                               round16<IS_BF16>(v[4 * a + 3] + b4[cb][a][3])};
              if (live)
                *reinterpret_cast<half4*>(out + static_cast<int64_t>(ORD[rb]) * COUT + 64 * w +
                                          32 * cb + 8 * a + 4 * h) = o;
            }
          acc[rb][0] = acc[rb][1] = float16v{};
        }
      }
      lds_barrier();  // the next slice and table are in place; this buffer is free
      sb ^= 1;
    }
    ib ^= 1;
    if (!has_next) break;
    ju = ju_n;
    d = d_n;
  }
}

template <int CIN, bool IS_BF16>
int launch_wide(const Map& m, const _Float16* feats, const _Float16* wp, const float* bias,
                _Float16* out, hipStream_t stream) {
  const Staged& S = m.staged;
  if (S.n_units > (int64_t{1} << 28))
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "too many staged units");
  int dev = 0, cus = 256;
  SUBMCONV_HIP_CHECK(hipGetDevice(&dev));
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int per_xcd = static_cast<int>((S.n_units + 7) / 8);
  const int slots = cus < 8 ? 1 : cus / 8;  // one workgroup per CU, dealt evenly to the XCDs
  const int wpx = per_xcd < slots ? per_xcd : slots;
  k_fwd_staged_wide<CIN, 256, IS_BF16><<<static_cast<unsigned>(8 * wpx), CfgW<CIN, 256>::NT, 0,
                                          stream>>>(
      S.units, static_cast<int>(S.n_units), per_xcd, wpx, S.rows,
      reinterpret_cast<const uint32_t*>(S.idx), staged_idx_stride(m.n) / 2, m.order, m.n, feats,
      wp, bias, out);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

}  // namespace

int forward_staged_wide(const Map& m, int cin, bool bf16, const _Float16* feats,
                        const _Float16* wp, const float* bias, _Float16* out,
                        hipStream_t stream) {
  if (cin == 256)
    return bf16 ? launch_wide<256, true>(m, feats, wp, bias, out, stream)
                : launch_wide<256, false>(m, feats, wp, bias, out, stream);
  if (cin == 128)
    return bf16 ? launch_wide<128, true>(m, feats, wp, bias, out, stream)
                : launch_wide<128, false>(m, feats, wp, bias, out, stream);
  return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "staged forward: 128 or 256 input channels");
}

}  // namespace submconv
