// Masked implicit-GEMM variant of the SubMConv3d forward on gfx950.
//
// The "masked implicit GEMM" of the trellis-mac issue #1 thread ("Fixed"
// list and its dense-vs-masked table): rows are grouped by which taps they
// use, and a block of rows runs the taps that at least one of its rows uses
// (the thread's skip-empty-V vote), every row of the block taking part with
// zeros where its neighbour is absent. The thread's precomputed structures
// map to this plan as: sorted_idx -> the rows sorted by their 27-bit
// neighbour mask; valid_kernel / valid_kernel_seg -> per block of kBlockRows
// sorted rows, the list of taps in the union of the block's masks and its
// offset.
//
// Unlike the in-tile compaction of k_fwd_pp, a block's rows are fixed for
// all its taps, so the fp32 accumulators stay in MFMA registers (no LDS
// accumulator); the price is the padding of each tap to the whole block.
// One workgroup = one block of 64 sorted rows x COUT_T columns; per tap the
// 64 neighbour rows are gathered into LDS (double buffered) and each wave
// multiplies them with its 32 columns of W[tap] on v_mfma_f32_32x32x16_f16.
#include <rocprim/device/device_radix_sort.hpp>
#include <rocprim/device/device_scan.hpp>

#include <type_traits>
#include <utility>

#include "submconv_internal.h"

namespace submconv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kBlockRows = 64;

// Two allocations: `head` holds rows, slot_off and the build's temporaries
// (sized before the build), `tail` the slot arrays (sized by the scan).
struct MaskedPlan {
  int device = 0;
  int64_t n = 0;
  int64_t n_blocks = 0;
  int64_t n_slots = 0;         // sum over blocks of the taps they run
  void* head = nullptr;
  void* tail = nullptr;
  int32_t* rows = nullptr;     // [n_blocks * 64] caller row of each sorted row (-1 past n)
  int32_t* slot_off = nullptr; // [n_blocks + 1] first tap slot of each block
  int32_t* slot_tap = nullptr; // [n_slots] tap of each slot
  int32_t* slot_nbr = nullptr; // [n_slots][64] neighbour caller row of each block row, or -1
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
constexpr uint32_t kOob = 0x80000000u;
__device__ __forceinline__ half8 bload_h8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// mask[t] = bit k set when row t (processing order) has a neighbour at tap k
__global__ void k_masks(const int32_t* __restrict__ nbr, int64_t n, uint32_t* __restrict__ mask,
                        int32_t* __restrict__ idx) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= n) return;
  uint32_t m = 0;
  for (int k = 0; k < kTaps3; ++k) m |= (nbr[static_cast<int64_t>(k) * n + t] >= 0 ? 1u : 0u) << k;
  mask[t] = m;
  idx[t] = static_cast<int32_t>(t);
}

// per block of 64 sorted rows: union of the masks, its tap count, and the
// caller row of each sorted row
__global__ void k_block_union(const uint32_t* __restrict__ smask, const int32_t* __restrict__ sidx,
                              const int32_t* __restrict__ order, int64_t n, int64_t n_blocks,
                              uint32_t* __restrict__ umask, int32_t* __restrict__ cnt,
                              int32_t* __restrict__ rows) {
  const int64_t b = static_cast<int64_t>(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (b >= n_blocks) return;
  const int64_t s = b * kBlockRows + lane;
  uint32_t m = 0;
  int32_t row = -1;
  if (s < n) {
    m = smask[s];
    const int32_t t = sidx[s];
    row = order ? order[t] : t;
  }
  rows[s] = row;
  for (int off = 32; off > 0; off >>= 1) m |= __shfl_xor(m, off, 64);
  if (lane == 0) {
    umask[b] = m;
    cnt[b] = __popc(m);
  }
}

// slot table: for each block and each tap of its union (ascending taps), the
// tap and the 64 neighbour caller rows
__global__ void k_slots(const uint32_t* __restrict__ umask, const int32_t* __restrict__ slot_off,
                        const int32_t* __restrict__ sidx, const int32_t* __restrict__ nbr,
                        int64_t n, int64_t n_blocks, int32_t* __restrict__ slot_tap,
                        int32_t* __restrict__ slot_nbr) {
  const int64_t b = static_cast<int64_t>(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (b >= n_blocks) return;
  const int64_t s = b * kBlockRows + lane;
  const int32_t t = s < n ? sidx[s] : -1;
  uint32_t m = umask[b];
  int slot = slot_off[b];
  while (m) {
    const int k = __ffs(m) - 1;
    m &= m - 1;
    if (lane == 0) slot_tap[slot] = k;
    slot_nbr[static_cast<int64_t>(slot) * kBlockRows + lane] =
        t >= 0 ? nbr[static_cast<int64_t>(k) * n + t] : -1;
    ++slot;
  }
}

template <int CIN, int COUT_T>
__global__ __launch_bounds__(2 * COUT_T) void k_fwd_masked(
    const int32_t* __restrict__ rows, const int32_t* __restrict__ slot_off,
    const int32_t* __restrict__ slot_tap, const int32_t* __restrict__ slot_nbr, int64_t n,
    const _Float16* __restrict__ feats, const _Float16* __restrict__ wp,
    const float* __restrict__ bias, _Float16* __restrict__ out, int cout, int n_ct) {
  constexpr int NW = COUT_T / 32, NT = 64 * NW, KS = CIN / 16, RC = CIN / 8;
  constexpr int GCH = kBlockRows * RC;           // 16-byte chunks per gathered tap
  constexpr int CPT = GCH / NT;                  // chunks per thread
  static_assert(GCH % NT == 0, "chunk split");
  __shared__ half8 bt[2][GCH];

  const int blk = blockIdx.x / n_ct;
  const int ct = blockIdx.x - blk * n_ct;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int s32 = lane & 31, h = lane >> 5;
  const int c0 = ct * COUT_T, cwb = c0 + 32 * w;
  const int sl0 = slot_off[blk], sl1 = slot_off[blk + 1];
  const int ns = sl1 - sl0;

  const __amdgpu_buffer_rsrc_t rf = make_rsrc(feats, static_cast<uint32_t>(n * CIN * 2));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wp, static_cast<uint32_t>(kTaps3 * CIN * cout * 2));

  // loader: chunk c = tid + NT*i of the gathered tap is row c / RC, chunk c % RC
  int lrow[CPT], lpos[CPT];
  uint32_t lcol[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + NT * i;
    lrow[i] = c / RC;
    const int lc = c % RC;
    lcol[i] = static_cast<uint32_t>(lc * 16);
    lpos[i] = lrow[i] * RC + (lc ^ (lrow[i] & (RC - 1)));
  }
  auto load_rows = [&](int s, half8 (&D)[CPT]) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int j = s < ns ? slot_nbr[static_cast<int64_t>(sl0 + s) * kBlockRows + lrow[i]] : -1;
      D[i] = bload_h8(rf, j >= 0 ? static_cast<uint32_t>(j) * (CIN * 2) + lcol[i] : kOob);
    }
  };
  auto store_rows = [&](int slot, const half8 (&D)[CPT]) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) bt[slot][lpos[i]] = D[i];
  };
  auto load_a = [&](int s, half8 (&A)[KS]) {
    const int tap = s < ns ? slot_tap[sl0 + s] : 0;
    const uint32_t base =
        static_cast<uint32_t>(((tap * (cout / 32) + (cwb >> 5)) * KS) * 1024 + lane * 16);
#pragma unroll
    for (int st = 0; st < KS; ++st) A[st] = bload_h8(rw, s < ns ? base + st * 1024 : kOob);
  };
  // B fragments of row group g (rows 32g..32g+31) from a gathered tap
  auto read_b = [&](int slot, int g, half8 (&B)[KS]) {
    const int r = 32 * g + s32;
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const int lc = h * (CIN / 16) + st;
      B[st] = bt[slot][r * RC + (lc ^ (r & (RC - 1)))];
    }
  };

  // LDS writes of this wave are complete, then all waves meet; outstanding
  // global prefetches stay in flight across the barrier
  auto lds_barrier = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  float16v acc[2] = {float16v{}, float16v{}};
  half8 D[CPT], AW[2][KS], B[KS];
  load_rows(0, D);
  load_a(0, AW[0]);
  store_rows(0, D);
  load_rows(1, D);
  lds_barrier();
  // tap slot s (its rows in LDS slot s%2, its weights in AW[s%2]): store the
  // rows of s+1, request the rows of s+2 and the weights of s+1, multiply s
  auto step = [&](int s, auto cc) {
    constexpr int cur = decltype(cc)::value;
    store_rows(cur ^ 1, D);
    load_rows(s + 2, D);
    load_a(s + 1, AW[cur ^ 1]);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      read_b(cur, g, B);
#pragma unroll
      for (int st = 0; st < KS; ++st)
        acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(AW[cur][st], B[st], acc[g], 0, 0, 0);
    }
    lds_barrier();
  };
  for (int s = 0; s < ns; s += 2) {
    step(s, std::integral_constant<int, 0>{});
    if (s + 1 < ns) step(s + 1, std::integral_constant<int, 1>{});
  }
  // epilogue: lane holds row 32g + lane%32 and columns 8a + 4h + b in
  // register 4a + b; bias in fp32, one rounding, 8-byte stores
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int row = rows[static_cast<int64_t>(blk) * kBlockRows + 32 * g + s32];
    if (row < 0) continue;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int col = cwb + 8 * a + 4 * h;
      _Float16 v[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        v[b] = static_cast<_Float16>(acc[g][4 * a + b] + (bias ? bias[col + b] : 0.f));
      typedef _Float16 half4 __attribute__((ext_vector_type(4)));
      *reinterpret_cast<half4*>(out + static_cast<int64_t>(row) * cout + col) =
          half4{v[0], v[1], v[2], v[3]};
    }
  }
}

void free_masked(MaskedPlan* d) {
  if (!d) return;
  if (d->head) (void)hipFree(d->head);
  if (d->tail) (void)hipFree(d->tail);
  delete d;
}

size_t up256(size_t v) { return (v + 255) & ~size_t{255}; }

template <int CIN, int COUT_T>
int launch_masked(const MaskedPlan& p, const _Float16* feats, const _Float16* wp, const float* bias,
                  _Float16* out, int cout, hipStream_t stream) {
  const int n_ct = cout / COUT_T;
  const int64_t blocks = p.n_blocks * n_ct;
  if (blocks > INT32_MAX) return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "too many blocks");
  k_fwd_masked<CIN, COUT_T><<<static_cast<unsigned>(blocks), 2 * COUT_T, 0, stream>>>(
      p.rows, p.slot_off, p.slot_tap, p.slot_nbr, p.n, feats, wp, bias, out, cout, n_ct);
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

template <int CIN>
int dispatch_masked(const MaskedPlan& p, const _Float16* feats, const _Float16* wp,
                    const float* bias, _Float16* out, int cout, hipStream_t stream) {
  if (cout % 128 == 0) return launch_masked<CIN, 128>(p, feats, wp, bias, out, cout, stream);
  if (cout % 64 == 0) return launch_masked<CIN, 64>(p, feats, wp, bias, out, cout, stream);
  return launch_masked<CIN, 32>(p, feats, wp, bias, out, cout, stream);
}

}  // namespace
}  // namespace submconv

struct submconv_masked_s {
  submconv::MaskedPlan p;
};

using namespace submconv;

#define MPLAN_CHECK(expr)                                                                    \
  do {                                                                                       \
    hipError_t e_ = (expr);                                                                  \
    if (e_ != hipSuccess) {                                                                  \
      free_masked(d);                                                                        \
      return set_error(e_ == hipErrorOutOfMemory ? SUBMCONV_ERR_OUT_OF_MEMORY : SUBMCONV_ERR_HIP, \
                       "%s failed: %s", #expr, hipGetErrorString(e_));                       \
    }                                                                                        \
  } while (0)

extern "C" int submconv_masked_plan(submconv_map_t map, hipStream_t stream,
                                    submconv_masked_t* out_plan) {
  clear_error();
  if (!map || !out_plan) return set_error(SUBMCONV_ERR_INVALID_ARG, "NULL argument");
  *out_plan = nullptr;
  const Map& m = map->m;
  MaskedPlan* d = new MaskedPlan;
  MPLAN_CHECK(hipGetDevice(&d->device));
  d->n = m.n;
  if (m.n == 0) {
    *out_plan = new submconv_masked_s{*d};
    delete d;
    return SUBMCONV_OK;
  }
  const int64_t n = m.n;
  d->n_blocks = (n + kBlockRows - 1) / kBlockRows;
  const size_t nn = static_cast<size_t>(n), nb = static_cast<size_t>(d->n_blocks);
  size_t sort_bytes = 0, scan_bytes = 0;
  MPLAN_CHECK(rocprim::radix_sort_pairs(nullptr, sort_bytes, static_cast<uint32_t*>(nullptr),
                                        static_cast<uint32_t*>(nullptr), static_cast<int32_t*>(nullptr),
                                        static_cast<int32_t*>(nullptr), nn, 0u,
                                        static_cast<unsigned>(kTaps3), stream));
  MPLAN_CHECK(rocprim::exclusive_scan(nullptr, scan_bytes, static_cast<int32_t*>(nullptr),
                                      static_cast<int32_t*>(nullptr), 0, nb + 1, rocprim::plus<int32_t>(),
                                      stream));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += up256(bytes > 0 ? bytes : 1);
    return o;
  };
  const size_t o_rows = take(4 * nb * kBlockRows), o_soff = take(4 * (nb + 1));
  const size_t o_mask = take(4 * nn), o_smask = take(4 * nn), o_idx = take(4 * nn), o_sidx = take(4 * nn);
  const size_t o_umask = take(4 * nb), o_cnt = take(4 * (nb + 1));
  const size_t o_sort = take(sort_bytes), o_scan = take(scan_bytes);
  MPLAN_CHECK(hipMalloc(&d->head, off));
  char* base = static_cast<char*>(d->head);
  d->rows = reinterpret_cast<int32_t*>(base + o_rows);
  d->slot_off = reinterpret_cast<int32_t*>(base + o_soff);
  uint32_t* mask = reinterpret_cast<uint32_t*>(base + o_mask);
  uint32_t* smask = reinterpret_cast<uint32_t*>(base + o_smask);
  int32_t* idx = reinterpret_cast<int32_t*>(base + o_idx);
  int32_t* sidx = reinterpret_cast<int32_t*>(base + o_sidx);
  uint32_t* umask = reinterpret_cast<uint32_t*>(base + o_umask);
  int32_t* cnt = reinterpret_cast<int32_t*>(base + o_cnt);
  const unsigned gb = static_cast<unsigned>((n + 255) / 256);
  k_masks<<<gb, 256, 0, stream>>>(m.nbr, n, mask, idx);
  MPLAN_CHECK(hipGetLastError());
  MPLAN_CHECK(rocprim::radix_sort_pairs(base + o_sort, sort_bytes, mask, smask, idx, sidx, nn, 0u,
                                        static_cast<unsigned>(kTaps3), stream));
  MPLAN_CHECK(hipMemsetAsync(cnt, 0, 4 * (nb + 1), stream));
  const unsigned gbb = static_cast<unsigned>((d->n_blocks + 3) / 4);
  k_block_union<<<gbb, 256, 0, stream>>>(smask, sidx, m.order, n, d->n_blocks, umask, cnt, d->rows);
  MPLAN_CHECK(hipGetLastError());
  MPLAN_CHECK(rocprim::exclusive_scan(base + o_scan, scan_bytes, cnt, d->slot_off, 0, nb + 1,
                                      rocprim::plus<int32_t>(), stream));
  int32_t total = 0;
  MPLAN_CHECK(hipMemcpyAsync(&total, d->slot_off + d->n_blocks, 4, hipMemcpyDeviceToHost, stream));
  MPLAN_CHECK(hipStreamSynchronize(stream));
  d->n_slots = total;
  const size_t ns = static_cast<size_t>(total > 0 ? total : 1);
  const size_t t_nbr = up256(4 * ns);
  MPLAN_CHECK(hipMalloc(&d->tail, t_nbr + 4 * kBlockRows * ns));
  d->slot_tap = static_cast<int32_t*>(d->tail);
  d->slot_nbr = reinterpret_cast<int32_t*>(static_cast<char*>(d->tail) + t_nbr);
  k_slots<<<gbb, 256, 0, stream>>>(umask, d->slot_off, sidx, m.nbr, n, d->n_blocks, d->slot_tap,
                                   d->slot_nbr);
  MPLAN_CHECK(hipGetLastError());
  MPLAN_CHECK(hipStreamSynchronize(stream));
  *out_plan = new submconv_masked_s{*d};
  delete d;
  return SUBMCONV_OK;
}

extern "C" int64_t submconv_masked_row_taps(submconv_masked_t plan) {
  if (!plan) return set_error(SUBMCONV_ERR_INVALID_ARG, "plan is NULL");
  return plan->p.n_slots * kBlockRows;
}

extern "C" int submconv_forward_masked(submconv_masked_t plan, const uint16_t* feats,
                                       submconv_weights_t wh, const float* bias, uint16_t* out,
                                       hipStream_t stream) {
  clear_error();
  if (!plan || !wh) return set_error(SUBMCONV_ERR_INVALID_ARG, "plan or weights is NULL");
  const MaskedPlan& p = plan->p;
  const Weights& W = wh->w;
  const int cin = W.cin, cout = W.cout;
  if (W.ksize != 3 || W.dtype != SUBMCONV_DTYPE_F16 || (W.flags & SUBMCONV_PREP_INPUT_GRAD))
    return set_error(SUBMCONV_ERR_INVALID_ARG,
                     "masked forward: the weights must be fp16, 3x3x3, prepared for the forward");
  // the shapes whose prepared weights are in MFMA fragment order
  if (!(((cin == 32 || cin == 64 || cin == 128) && cout % 32 == 0) || (cin == 256 && cout % 128 == 0)) ||
      cout > 1024)
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE,
                     "masked forward: Cin in {32, 64, 128} with Cout a multiple of 32, or Cin 256 "
                     "with Cout a multiple of 128 (got %d, %d)", cin, cout);
  if (p.n == 0) return SUBMCONV_OK;
  if (!feats || !out) return set_error(SUBMCONV_ERR_INVALID_ARG, "feats or out is NULL");
  if ((reinterpret_cast<uintptr_t>(feats) | reinterpret_cast<uintptr_t>(out) |
       reinterpret_cast<uintptr_t>(bias)) & 15)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "feats, out and bias must be 16-byte aligned");
  int dev = -1;
  SUBMCONV_HIP_CHECK(hipGetDevice(&dev));
  if (dev != W.device || dev != p.device)
    return set_error(SUBMCONV_ERR_INVALID_ARG,
                     "plan (device %d), weights (device %d) and the current device (%d) differ",
                     p.device, W.device, dev);
  if (p.n * cin * 2 >= (int64_t{1} << 31) - 64)
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "features beyond 2 GiB");
  const _Float16* f = reinterpret_cast<const _Float16*>(feats);
  const _Float16* w = W.buf;
  _Float16* o = reinterpret_cast<_Float16*>(out);
  switch (cin) {
    case 32: return dispatch_masked<32>(p, f, w, bias, o, cout, stream);
    case 64: return dispatch_masked<64>(p, f, w, bias, o, cout, stream);
    case 128: return dispatch_masked<128>(p, f, w, bias, o, cout, stream);
    default: return dispatch_masked<256>(p, f, w, bias, o, cout, stream);
  }
}

extern "C" int submconv_masked_free(submconv_masked_t plan) {
  if (!plan) return SUBMCONV_OK;
  MaskedPlan* d = new MaskedPlan(plan->p);
  delete plan;
  free_masked(d);
  return SUBMCONV_OK;
}
