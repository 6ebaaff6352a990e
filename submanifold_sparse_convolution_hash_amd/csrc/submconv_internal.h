// Internal declarations shared by the map builder and the forward kernels of
// libsubmconv.so. Not part of the public ABI (include/submconv.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/submconv.h"

namespace submconv {

// Number of taps of a 3x3x3 kernel and the centre tap, k = 9(dx+1)+3(dy+1)+(dz+1).
constexpr int kTaps3 = 27;
constexpr int kCenterTap = 13;

// Rows per output tile of the forward kernels; the map's per-tile lists are
// built for this tile size, or for up to kTileRowsWide rows (Map.tile_rows)
// when that spreads a sparse map more evenly over the compute units.
constexpr int kTileRows = 256;
constexpr int kTileRowsWide = 288;

// Entries per group: the kernels take a tile's entries of one position 32
// at a time (one MFMA operand block).
constexpr int kGroupRows = 32;

// Processing position p -> tap: the centre first (it initialises an output
// accumulator), then the other 26 taps in ascending order.
__host__ __device__ inline int tap_at(int p) {
  return p == 0 ? kCenterTap : (p <= kCenterTap ? p - 1 : p);
}

// Kernel map: library-owned, immutable after the build.
//  nbr      [27][n] int32, tap-major, rows in processing order t; each entry
//           is the caller row of the neighbour at offset d_k, or -1.
//  order    [n] int32, processing order t -> caller row; nullptr = identity.
//  tiles    the same map as per-tile compacted lists of kTileRows-row
//           tiles, the form the forward kernels stream;
//  wide     for sparse maps, the lists of tiles of up to kTileRowsWide rows
//           as well (wide.n == 0: none); a forward takes them when they fit
//           its workgroups into fewer rounds.
// One tiling (tiles of `rows` consecutive processing rows):
//  cnt  [n][27] uint16, entries per processing position p.
//  off  [n + 1] int32, first entry of each tile.
//  ent  [active_pairs + 1] int2 {caller row of the neighbour, row in tile},
//       ordered by (tile, position p, row in tile), then one entry {-1, -1}
//       that masked lanes load instead of selecting -1.
struct Tiles {
  int32_t rows = kTileRows;
  int64_t n = 0;
  uint16_t* cnt = nullptr;
  int32_t* off = nullptr;
  int2* ent = nullptr;
  // groups of kGroupRows entries per processing position, over all tiles
  int64_t pos_groups[kTaps3] = {};
};
struct Map {
  int device = 0;
  int64_t n = 0;
  int32_t batch = 1;
  int32_t grid[3] = {0, 0, 0};
  uint32_t flags = 0;
  int64_t active_pairs = 0;
  // two device allocations hold everything below: `mem` the neighbour table,
  // the order and both tile sets' counts and offsets, `ent_mem` the lists
  void* mem = nullptr;
  void* ent_mem = nullptr;
  int32_t* nbr = nullptr;
  int32_t* order = nullptr;
  Tiles tiles;
  Tiles wide;
  bool wide_always = false;  // forwards take the wide tiles whenever their kernel can
};

// Records a thread-local message and returns `status`.
int set_error(int status, const char* fmt, ...);
void clear_error();
const char* last_error_cstr();

}  // namespace submconv

struct submconv_map_s {
  submconv::Map m;
};

#define SUBMCONV_HIP_CHECK(expr)                                                              \
  do {                                                                                        \
    hipError_t e_ = (expr);                                                                   \
    if (e_ != hipSuccess)                                                                     \
      return ::submconv::set_error(e_ == hipErrorOutOfMemory ? SUBMCONV_ERR_OUT_OF_MEMORY     \
                                                             : SUBMCONV_ERR_HIP,              \
                                   "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_),    \
                                   __FILE__, __LINE__);                                       \
  } while (0)
