// x2 downsample (max-pool) and x2 subdivide of a sparse tensor on gfx950:
// the coordinate operations next to SubMConv3d in the same sparse stack
// (trellis_sparse_mlx README, "What's in it" table, subdivide / downsample
// row: x2 coordinate expansion, and x2 max-pooling with the "amax" reduce).
//
// Downsample: every site's parent key ((b*P0 + x/2)*P1 + y/2)*P2 + z/2
// (P = parent grid) is radix sorted with the site index; equal keys are
// adjacent, so the parents are the distinct keys in ascending order (the
// order of a sorting unique) and each parent's children are one contiguous
// run of the sorted indices. A plan keeps the runs; the parent features are
// then a max over each run, for any number of feature tensors.
//
// Subdivide: site i becomes rows 8i + c, c = 4dx + 2dy + dz, at
// (b, 2x+dx, 2y+dy, 2z+dz), each with site i's features.
#include <rocprim/device/device_radix_sort.hpp>
#include <rocprim/device/device_scan.hpp>

#include "submconv_internal.h"

namespace submconv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

// All of a plan's device arrays, and the temporaries its build uses, live in
// one allocation (blob): a build costs one hipMalloc and a release one hipFree.
struct DownPlan {
  int device = 0;
  int64_t n = 0, m = 0;
  int32_t pgrid[3] = {0, 0, 0};
  void* blob = nullptr;
  int32_t* sorted_child = nullptr;  // [n] site indices in parent-key order
  int32_t* seg = nullptr;           // [m+1] run of parent p: sorted_child[seg[p] .. seg[p+1])
  int32_t* inverse = nullptr;       // [n] parent row of each site (the sort's index input first)
  int32_t* pcoords = nullptr;       // [m][4]
};

// K is uint32_t when batch * P0 * P1 * P2 fits in 32 bits (the radix sort then
// moves half the key bytes), else uint64_t.
template <typename K>
__global__ void k_parent_keys(const int32_t* __restrict__ coords, int64_t n, int32_t batch,
                              int32_t g0, int32_t g1, int32_t g2, int32_t p0, int32_t p1,
                              int32_t p2, K* __restrict__ keys, int32_t* __restrict__ idx,
                              uint32_t* __restrict__ err) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t b = coords[4 * i], x = coords[4 * i + 1], y = coords[4 * i + 2], z = coords[4 * i + 3];
  if (b < 0 || b >= batch || x < 0 || x >= g0 || y < 0 || y >= g1 || z < 0 || z >= g2) {
    atomicOr(err, 1u);
    keys[i] = 0;
  } else {
    keys[i] = ((static_cast<K>(b) * static_cast<K>(p0) + static_cast<K>(x >> 1)) * static_cast<K>(p1) +
               static_cast<K>(y >> 1)) * static_cast<K>(p2) + static_cast<K>(z >> 1);
  }
  idx[i] = static_cast<int32_t>(i);
}

// 1 where a new parent key starts in the sorted order
template <typename K>
__global__ void k_run_heads(const K* __restrict__ skeys, int64_t n, int32_t* __restrict__ head) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t < n) head[t] = (t == 0 || skeys[t] != skeys[t - 1]) ? 1 : 0;
}

// pos[t] = exclusive scan of head: parent row of sorted position t is
// pos[t] + head[t] - 1. The last position also writes the parent count M to
// *count, so the host reads M and the range flag in one copy.
template <typename K>
__global__ void k_runs(const K* __restrict__ skeys, const int32_t* __restrict__ schild,
                       const int32_t* __restrict__ head, const int32_t* __restrict__ pos, int64_t n,
                       int32_t p0, int32_t p1, int32_t p2, int32_t* __restrict__ seg,
                       int32_t* __restrict__ inverse, int32_t* __restrict__ pcoords,
                       uint32_t* __restrict__ count) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const int32_t p = pos[t] + head[t] - 1;
  inverse[schild[t]] = p;
  if (head[t]) {
    seg[p] = static_cast<int32_t>(t);
    K k = skeys[t];
    const int32_t z = static_cast<int32_t>(k % static_cast<K>(p2));
    k /= static_cast<K>(p2);
    const int32_t y = static_cast<int32_t>(k % static_cast<K>(p1));
    k /= static_cast<K>(p1);
    const int32_t x = static_cast<int32_t>(k % static_cast<K>(p0));
    const int32_t b = static_cast<int32_t>(k / static_cast<K>(p0));
    pcoords[4 * p] = b;
    pcoords[4 * p + 1] = x;
    pcoords[4 * p + 2] = y;
    pcoords[4 * p + 3] = z;
  }
  if (t == n - 1) {
    seg[p + 1] = static_cast<int32_t>(n);
    *count = static_cast<uint32_t>(p + 1);
  }
}

// parent p, 8-channel chunk c8: max over the run of p (fp16 max is exact)
__global__ void k_down_max(const int32_t* __restrict__ sorted_child, const int32_t* __restrict__ seg,
                           int64_t m, const _Float16* __restrict__ feats, int32_t cdim,
                           _Float16* __restrict__ out) {
  const int c8n = cdim / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= m * c8n) return;
  const int64_t p = idx / c8n;
  const int c8 = static_cast<int>(idx - p * c8n);
  const int32_t s0 = seg[p], s1 = seg[p + 1];
  half8 mx = *reinterpret_cast<const half8*>(feats + static_cast<int64_t>(sorted_child[s0]) * cdim + 8 * c8);
  for (int32_t s = s0 + 1; s < s1; ++s) {
    const half8 v =
        *reinterpret_cast<const half8*>(feats + static_cast<int64_t>(sorted_child[s]) * cdim + 8 * c8);
#pragma unroll
    for (int q = 0; q < 8; ++q) mx[q] = v[q] > mx[q] ? v[q] : mx[q];
  }
  *reinterpret_cast<half8*>(out + p * cdim + 8 * c8) = mx;
}

__global__ void k_subdivide(const int32_t* __restrict__ coords, int64_t n,
                            const _Float16* __restrict__ feats, int32_t cdim,
                            int32_t* __restrict__ ocoords, _Float16* __restrict__ ofeats) {
  const int c8n = feats ? cdim / 8 : 0;
  const int per = 8 * (1 + c8n);  // work items per site: 8 coordinate rows + 8 x c8n chunks
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n * per) return;
  const int64_t i = idx / per;
  const int r = static_cast<int>(idx - i * per);
  if (r < 8) {
    const int dx = r >> 2, dy = (r >> 1) & 1, dz = r & 1;
    int32_t* o = ocoords + 4 * (8 * i + r);
    o[0] = coords[4 * i];
    o[1] = 2 * coords[4 * i + 1] + dx;
    o[2] = 2 * coords[4 * i + 2] + dy;
    o[3] = 2 * coords[4 * i + 3] + dz;
  } else {
    const int q = r - 8;
    const int c = q / c8n, c8 = q - c * c8n;
    *reinterpret_cast<half8*>(ofeats + (8 * i + c) * cdim + 8 * c8) =
        *reinterpret_cast<const half8*>(feats + i * cdim + 8 * c8);
  }
}

int bits_of(uint64_t v) {  // bits to hold values < v
  int b = 1;
  while (b < 64 && (uint64_t{1} << b) < v) ++b;
  return b;
}

void free_plan(DownPlan* d) {
  if (!d) return;
  if (d->blob) (void)hipFree(d->blob);
  delete d;
}

size_t up256(size_t v) { return (v + 255) & ~size_t{255}; }

// Carves the plan's arrays and the build's temporaries out of one
// allocation, sorts the parent keys, and marks the runs. Returns the HIP
// error of the first failing call; *flags receives {range flag, M}.
template <typename K>
hipError_t build_plan(DownPlan* d, const int32_t* coords, int32_t batch, const int32_t grid[3],
                      uint64_t span, hipStream_t stream, uint32_t flags[2]) {
  const int64_t n = d->n;
  const size_t nn = static_cast<size_t>(n);
  const int end_bit = bits_of(span);
  size_t sort_bytes = 0, scan_bytes = 0;
  hipError_t e = rocprim::radix_sort_pairs(nullptr, sort_bytes, static_cast<K*>(nullptr),
                                           static_cast<K*>(nullptr), static_cast<int32_t*>(nullptr),
                                           static_cast<int32_t*>(nullptr), nn, 0, end_bit, stream);
  if (e != hipSuccess) return e;
  e = rocprim::exclusive_scan(nullptr, scan_bytes, static_cast<int32_t*>(nullptr),
                              static_cast<int32_t*>(nullptr), 0, nn, rocprim::plus<int32_t>(), stream);
  if (e != hipSuccess) return e;
  // offsets: plan arrays first, then the temporaries
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += up256(bytes > 0 ? bytes : 1);
    return o;
  };
  const size_t o_child = take(4 * nn), o_inv = take(4 * nn), o_seg = take(4 * (nn + 1));
  const size_t o_pc = take(16 * nn), o_keys = take(sizeof(K) * nn), o_skeys = take(sizeof(K) * nn);
  const size_t o_head = take(4 * nn), o_pos = take(4 * nn), o_small = take(16);
  const size_t o_sort = take(sort_bytes), o_scan = take(scan_bytes);
  e = hipMalloc(&d->blob, off);
  if (e != hipSuccess) return e;
  char* base = static_cast<char*>(d->blob);
  d->sorted_child = reinterpret_cast<int32_t*>(base + o_child);
  d->inverse = reinterpret_cast<int32_t*>(base + o_inv);
  d->seg = reinterpret_cast<int32_t*>(base + o_seg);
  d->pcoords = reinterpret_cast<int32_t*>(base + o_pc);
  K* keys = reinterpret_cast<K*>(base + o_keys);
  K* skeys = reinterpret_cast<K*>(base + o_skeys);
  int32_t* head = reinterpret_cast<int32_t*>(base + o_head);
  int32_t* pos = reinterpret_cast<int32_t*>(base + o_pos);
  uint32_t* small = reinterpret_cast<uint32_t*>(base + o_small);
  // the sort's index input lives in inverse: it is dead once the sort has run
  int32_t* idx = d->inverse;
  e = hipMemsetAsync(small, 0, 16, stream);
  if (e != hipSuccess) return e;
  const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
  k_parent_keys<K><<<blocks, 256, 0, stream>>>(coords, n, batch, grid[0], grid[1], grid[2], d->pgrid[0],
                                               d->pgrid[1], d->pgrid[2], keys, idx, small);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = rocprim::radix_sort_pairs(base + o_sort, sort_bytes, keys, skeys, idx, d->sorted_child, nn, 0,
                                end_bit, stream);
  if (e != hipSuccess) return e;
  k_run_heads<K><<<blocks, 256, 0, stream>>>(skeys, n, head);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = rocprim::exclusive_scan(base + o_scan, scan_bytes, head, pos, 0, nn, rocprim::plus<int32_t>(),
                              stream);
  if (e != hipSuccess) return e;
  k_runs<K><<<blocks, 256, 0, stream>>>(skeys, d->sorted_child, head, pos, n, d->pgrid[0], d->pgrid[1],
                                        d->pgrid[2], d->seg, d->inverse, d->pcoords, small + 1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = hipMemcpyAsync(flags, small, 8, hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(stream);
}

}  // namespace
}  // namespace submconv

struct submconv_down_s {
  submconv::DownPlan d;
};

using namespace submconv;

extern "C" int submconv_downsample_plan(const int32_t* coords, int64_t n, int32_t batch,
                                        const int32_t grid[3], hipStream_t stream,
                                        submconv_down_t* out_plan) {
  clear_error();
  if (!out_plan) return set_error(SUBMCONV_ERR_INVALID_ARG, "out_plan is NULL");
  *out_plan = nullptr;
  if (n < 0 || batch < 1 || !grid || (n > 0 && !coords))
    return set_error(SUBMCONV_ERR_INVALID_ARG, "bad arguments");
  if (grid[0] < 1 || grid[1] < 1 || grid[2] < 1)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "grid extents must be positive");
  if (n >= INT32_MAX) return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "too many sites");
  DownPlan* d = new DownPlan;
  hipError_t e = hipGetDevice(&d->device);
  d->n = n;
  for (int a = 0; a < 3; ++a) d->pgrid[a] = (grid[a] + 1) / 2;
  const uint64_t span = static_cast<uint64_t>(batch) * d->pgrid[0] * d->pgrid[1] * d->pgrid[2];
  uint32_t flags[2] = {0, 0};
  if (e == hipSuccess && n > 0)
    e = span <= (uint64_t{1} << 32) ? build_plan<uint32_t>(d, coords, batch, grid, span, stream, flags)
                                    : build_plan<uint64_t>(d, coords, batch, grid, span, stream, flags);
  if (e != hipSuccess) {
    free_plan(d);
    return set_error(e == hipErrorOutOfMemory ? SUBMCONV_ERR_OUT_OF_MEMORY : SUBMCONV_ERR_HIP,
                     "downsample plan: %s", hipGetErrorString(e));
  }
  if (flags[0]) {
    free_plan(d);
    return set_error(SUBMCONV_ERR_COORD_OUT_OF_RANGE, "a site lies outside [0,%d) x [0,%d) x [0,%d) x [0,%d)",
                     batch, grid[0], grid[1], grid[2]);
  }
  d->m = n > 0 ? static_cast<int64_t>(flags[1]) : 0;
  *out_plan = new submconv_down_s{*d};
  delete d;
  return SUBMCONV_OK;
}

extern "C" int64_t submconv_downsample_rows(submconv_down_t plan) {
  if (!plan) return set_error(SUBMCONV_ERR_INVALID_ARG, "plan is NULL");
  return plan->d.m;
}

extern "C" int submconv_downsample_grid(submconv_down_t plan, int32_t pgrid[3]) {
  if (!plan || !pgrid) return set_error(SUBMCONV_ERR_INVALID_ARG, "NULL argument");
  for (int a = 0; a < 3; ++a) pgrid[a] = plan->d.pgrid[a];
  return SUBMCONV_OK;
}

extern "C" int submconv_downsample_coords(submconv_down_t plan, int32_t* pcoords, int32_t* inverse,
                                          hipStream_t stream) {
  clear_error();
  if (!plan) return set_error(SUBMCONV_ERR_INVALID_ARG, "plan is NULL");
  const DownPlan& d = plan->d;
  if (d.n == 0) return SUBMCONV_OK;
  if (pcoords)
    SUBMCONV_HIP_CHECK(hipMemcpyAsync(pcoords, d.pcoords, sizeof(int32_t) * 4 * d.m,
                                      hipMemcpyDeviceToDevice, stream));
  if (inverse)
    SUBMCONV_HIP_CHECK(hipMemcpyAsync(inverse, d.inverse, sizeof(int32_t) * d.n,
                                      hipMemcpyDeviceToDevice, stream));
  return SUBMCONV_OK;
}

extern "C" int submconv_downsample_max(submconv_down_t plan, const uint16_t* feats, int32_t cdim,
                                       uint16_t* out, hipStream_t stream) {
  clear_error();
  if (!plan) return set_error(SUBMCONV_ERR_INVALID_ARG, "plan is NULL");
  if (cdim <= 0 || cdim % 8 || cdim > 4096)
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "C = %d must be a positive multiple of 8", cdim);
  const DownPlan& d = plan->d;
  if (d.n == 0) return SUBMCONV_OK;
  if (!feats || !out) return set_error(SUBMCONV_ERR_INVALID_ARG, "feats or out is NULL");
  if ((reinterpret_cast<uintptr_t>(feats) | reinterpret_cast<uintptr_t>(out)) & 15)
    return set_error(SUBMCONV_ERR_INVALID_ARG, "feats and out must be 16-byte aligned");
  const int64_t items = d.m * (cdim / 8);
  k_down_max<<<static_cast<unsigned>((items + 255) / 256), 256, 0, stream>>>(
      d.sorted_child, d.seg, d.m, reinterpret_cast<const _Float16*>(feats), cdim,
      reinterpret_cast<_Float16*>(out));
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}

extern "C" int submconv_downsample_free(submconv_down_t plan) {
  if (!plan) return SUBMCONV_OK;
  DownPlan* d = new DownPlan(plan->d);
  delete plan;
  free_plan(d);
  return SUBMCONV_OK;
}

extern "C" int submconv_subdivide(const int32_t* coords, int64_t n, const uint16_t* feats,
                                  int32_t cdim, int32_t* out_coords, uint16_t* out_feats,
                                  hipStream_t stream) {
  clear_error();
  if (n < 0 || (n > 0 && (!coords || !out_coords)))
    return set_error(SUBMCONV_ERR_INVALID_ARG, "bad arguments");
  if (feats && (!out_feats || cdim <= 0 || cdim % 8 || cdim > 4096))
    return set_error(SUBMCONV_ERR_UNSUPPORTED_SHAPE, "C = %d must be a positive multiple of 8", cdim);
  if (feats && ((reinterpret_cast<uintptr_t>(feats) | reinterpret_cast<uintptr_t>(out_feats)) & 15))
    return set_error(SUBMCONV_ERR_INVALID_ARG, "feats and out_feats must be 16-byte aligned");
  if (n == 0) return SUBMCONV_OK;
  const int per = 8 * (1 + (feats ? cdim / 8 : 0));
  const int64_t items = n * per;
  k_subdivide<<<static_cast<unsigned>((items + 255) / 256), 256, 0, stream>>>(
      coords, n, reinterpret_cast<const _Float16*>(feats), cdim, out_coords,
      reinterpret_cast<_Float16*>(out_feats));
  SUBMCONV_HIP_CHECK(hipGetLastError());
  return SUBMCONV_OK;
}
