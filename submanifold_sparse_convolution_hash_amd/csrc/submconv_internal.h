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
//  cnt  [n_tiles][27] uint16, entries per processing position p.
//  off  [n_tiles + 1] int32, first entry of each tile.
//  ent  [active_pairs + 1] int2 {caller row of the neighbour, row in tile},
//       ordered by (tile, position p, row in tile), then one entry {-1, -1}
//       that masked lanes load instead of selecting -1.
struct Tiles {
  int32_t rows = kTileRows;
  int64_t n = 0;
  uint16_t* cnt = nullptr;
  int32_t* off = nullptr;
  int2* ent = nullptr;
  // [n] int32 or nullptr: the order in which each XCD's run of tiles is
  // walked (position i of the run -> tile), balanced across the workgroups
  // of a forward with one workgroup per CU; nullptr: tile i at position i
  int32_t* walk = nullptr;
  // groups of kGroupRows entries per processing position, over all tiles
  int64_t pos_groups[kTaps3] = {};
};
// Staged plan of a dense map (many neighbours per row): the rows cut into
// units of up to kStageUnitRows consecutive processing rows whose distinct
// neighbour rows over all 27 taps number at most kStageCap, so that a
// workgroup holds them in LDS and every tap reads them from there.
//  units  [n_units] int4 {first processing row, rows, first staged row,
//         staged rows}, in processing order;
//  rows   [n_rows] caller rows each unit stages, ascending within a unit;
//  idx    [27][stride] uint16, stride = n rounded up to even: the neighbour
//         of processing row t at tap k as a row of its unit's staged rows, or
//         kStageNone. Units start on even rows, so that a unit's entries of a
//         tap are whole 4-byte words.
// A tile of kStageUnitRows rows whose neighbours exceed kStageCap is halved
// until they fit; 27 * kStageMinRows <= kStageCap, so halves of at most
// kStageMinRows rows always do.
constexpr int kStageUnitRows = 128;
constexpr int kStageCap = 512;
constexpr int kStageMinRows = 16;
constexpr uint16_t kStageNone = 0xFFFF;
// mean neighbours per row (centre included) from which a build makes the
// staged plan
constexpr int kStageMinPairsPerRow = 12;
inline int64_t staged_idx_stride(int64_t n) { return n + (n & 1); }
constexpr int kStageMaxUnitsPerTile = 16;
struct Staged {
  int64_t n_units = 0;
  int64_t n_rows = 0;
  int4* units = nullptr;
  int32_t* rows = nullptr;
  uint16_t* idx = nullptr;
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
  // the staged plan (staged.n_units == 0: none), in its own allocation
  void* staged_mem = nullptr;
  Staged staged;
};

// Prepared weights of one layer (W [K][cin][cout]): the MFMA fragment order
// for shapes the MFMA kernels take, else W_t[k][ci][co] of the forward they
// serve (flipped and transposed under SUBMCONV_PREP_INPUT_GRAD).
struct Weights {
  int device = 0;
  int ksize = 3, cin = 0, cout = 0, dtype = SUBMCONV_DTYPE_F16;
  uint32_t flags = 0;
  _Float16* buf = nullptr;  // K * cin * cout elements, library-owned
};

// Build of the staged plan, in two passes around one host wait: the count
// pass splits the tiles into units and scans their sizes (totals[0] units,
// totals[1] staged rows); the fill pass, once the plan is allocated, writes it.
struct StagedTemps {
  int64_t n_tiles = 0;     // tiles of kStageUnitRows rows
  int4* tile_units = nullptr;  // [n_tiles][16] {row in tile, rows, staged rows, 0}
  int32_t* tile_nu = nullptr;  // [n_tiles] units of each tile
  int32_t* tile_ns = nullptr;  // [n_tiles] staged rows of each tile
  int64_t* unit_off = nullptr;   // [n_tiles] first unit of each tile
  int64_t* staged_off = nullptr; // [n_tiles] first staged row of each tile
  int64_t* totals = nullptr;     // [2]
};
int staged_count(const int32_t* nbr, int64_t n, const StagedTemps& tp, hipStream_t stream);
int staged_fill(const int32_t* nbr, int64_t n, const StagedTemps& tp, const Staged& plan,
                hipStream_t stream);

// The staged forward takes a 3x3x3 forward of 32 -> 32, 32 -> 64, 64 -> 32,
// 128 -> 256 or 256 -> 256 channels on a map with a staged plan (weights in
// MFMA fragment order); forward_staged_wide runs the 256-column shapes.
bool staged_shape(int cin, int cout);
bool staged_takes(const Map& m, int ksize, int cin, int cout);
int forward_staged(const Map& m, int cin, int cout, bool bf16, const _Float16* feats,
                   const _Float16* wp, const float* bias, _Float16* out, hipStream_t stream);
int forward_staged_wide(const Map& m, int cin, bool bf16, const _Float16* feats,
                        const _Float16* wp, const float* bias, _Float16* out,
                        hipStream_t stream);

// The staged weight gradient (3x3x3, fp16; 32 -> 32, 64 -> 32 or 32 -> 64
// channels on a map with a staged plan): its workgroups, each writing
// 27 x cin x cout fp32 partials (0 when it does not apply), and the call,
// which adds the partials into dw.
int64_t staged_wgrad_blocks(const Map& m, int ksize, int cin, int cout);
int backward_weight_staged(const Map& m, int cin, int cout, const _Float16* feats,
                           const _Float16* grad_out, float* partial, float* dw,
                           hipStream_t stream);

// Allocates the device's staging buffer for weights passed as the caller
// holds them (once per device; every map build calls it).
int ensure_weight_stage(int device);

// Records a thread-local message and returns `status`.
int set_error(int status, const char* fmt, ...);
void clear_error();
const char* last_error_cstr();

}  // namespace submconv

struct submconv_map_s {
  submconv::Map m;
};

struct submconv_weights_s {
  submconv::Weights w;
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
