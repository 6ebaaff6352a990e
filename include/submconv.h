/*
 * submconv.h -- C ABI of libsubmconv.so: submanifold sparse 3D convolution
 * (SubMConv3d, 3x3x3 and 1x1x1, stride 1) on AMD Instinct MI355X (gfx950).
 *
 * The operation (trellis_sparse_mlx README, "What's in it" table, SubMConv3d
 * and SparseTensor rows; "Performance" and "Correctness" sections):
 *
 *   A sparse tensor is a set of N distinct voxel sites coords[i] = (b,x,y,z)
 *   with a feature row feats[i] of Cin values. A submanifold convolution
 *   computes an output row only at the input sites:
 *
 *     out[i] = bias + sum over offsets d in {-1,0,1}^3 (or d = 0 for 1x1x1)
 *              of feats[j] @ W[k(d)],  where coords[j] = coords[i] + d,
 *
 *   with the gather at c + d (cross-correlation), the same batch item b, and
 *   absent neighbours (no site there, or outside the grid) contributing zero.
 *   Tap index k(dx,dy,dz) = 9(dx+1) + 3(dy+1) + (dz+1), dx slowest; the
 *   centre tap is k = 13. For a 1x1x1 kernel the single tap is k = 0.
 *
 * Work is split into a one-time kernel-map build per site set (a GPU hash of
 * the sites and the [N,27] neighbour map; the cached, device-resident gather
 * index of the README's "Performance" section) and a per-layer forward that
 * reuses it.
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers on the current HIP device unless
 *     marked "host". The caller owns them; the library never frees them.
 *   - fp16 data is passed as uint16_t holding IEEE-754 binary16 bit patterns.
 *   - Row-major, densely packed layouts; feature and weight pointers must be
 *     16-byte aligned.
 *   - Work is enqueued on `stream` (0 = the null stream) and, unless stated,
 *     returns without waiting for the device.
 *   - Return value: SUBMCONV_OK (0) or a negative status; argument and shape
 *     errors are detected before anything is enqueued. submconv_last_error()
 *     gives a thread-local message for the last failure.
 */
#ifndef SUBMCONV_H_
#define SUBMCONV_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SUBMCONV_ABI_VERSION 2

/* Status codes. */
#define SUBMCONV_OK 0
#define SUBMCONV_ERR_INVALID_ARG (-1)        /* NULL pointer, negative size, bad ksize */
#define SUBMCONV_ERR_COORD_OUT_OF_RANGE (-2) /* a site outside [0,batch) x grid */
#define SUBMCONV_ERR_DUPLICATE_COORD (-3)    /* the same site given twice */
#define SUBMCONV_ERR_UNSUPPORTED_SHAPE (-4)  /* Cin/Cout not multiples of 8, too large, ... */
#define SUBMCONV_ERR_HIP (-5)                /* a HIP runtime call or launch failed */
#define SUBMCONV_ERR_OUT_OF_MEMORY (-6)      /* device allocation failed */

/* Flags of submconv_build_map. */
#define SUBMCONV_FLAG_MORTON 1u /* process output rows in Morton (Z-curve) order */
/* find neighbours by binary search in the radix-sorted packed site keys
 * instead of the hash table (the packing + sort + search lookup of "Running
 * TRELLIS.2 on a Mac (3/3)", section E); the map is the same */
#define SUBMCONV_FLAG_SORTED_KEYS 2u
/* tile size of the per-tile neighbour lists the forward streams: the map
 * always holds lists of 256-row tiles; when it is sparse (under 32 entries
 * per off-centre tap and 256-row tile on average) and tiles of up to 288 rows
 * need fewer rounds of one tile per compute unit, it also holds lists of the
 * fewest rows (257..288) that fit the tiles into those rounds, and each
 * forward takes whichever fits its own workgroups into fewer rounds.
 * SUBMCONV_FLAG_TILES_256 builds no wider lists; SUBMCONV_FLAG_TILES_288
 * builds 288-row lists and makes every forward that can use them (the
 * results are the same bit for bit) */
#define SUBMCONV_FLAG_TILES_256 4u
#define SUBMCONV_FLAG_TILES_288 8u
/* the staged plan: on a dense map (at least 12 neighbours per row on
 * average, centre included, as on a surface) the build also cuts the rows
 * into units of up to 128 whose distinct neighbour rows (at most 512) a
 * forward of 32 -> 32, 64 -> 32, 32 -> 64, 128 -> 256 or 256 -> 256 channels
 * stages once in LDS, instead of gathering each (row, tap) pair (the input
 * gradient of such a shape too, when its transposed shape is one of them);
 * it costs 54 bytes per row plus 4 per staged
 * row. SUBMCONV_FLAG_STAGED builds it on any map, SUBMCONV_FLAG_NO_STAGED on
 * none (such forwards then take the compacted lists) */
#define SUBMCONV_FLAG_STAGED 16u
#define SUBMCONV_FLAG_NO_STAGED 32u

/* 16-bit element types of features and weights (the *_dtype entry points). */
#define SUBMCONV_DTYPE_F16 0  /* IEEE binary16 */
#define SUBMCONV_DTYPE_BF16 1 /* bfloat16 (the top 16 bits of a binary32) */

/* Flags of submconv_weights_create. */
#define SUBMCONV_PREP_INPUT_GRAD 1u /* prepare the flipped, transposed kernel of the input gradient */

/* Opaque kernel-map handle: library-owned device buffers, immutable after
 * submconv_build_map returns, released by submconv_map_free. One handle may
 * serve concurrent forwards on several streams of its device. */
typedef struct submconv_map_s* submconv_map_t;

/*
 * submconv_build_map -- hash the sites and build the neighbour map: the
 * cached gather index of the README's "Performance" section (a one-time cost
 * per site set that every layer on those sites reuses), for the sparse
 * tensor of its "What's in it" SparseTensor row (coords [N,4], batch index
 * first). It is a GPU coordinate hash where "Running TRELLIS.2 on a Mac
 * (3/3)", section E, replaces a Python dict of coordinates with injectively
 * packed int64 keys and a sorted search (which SUBMCONV_FLAG_SORTED_KEYS
 * builds as well).
 *
 * coords   [n,4] int32 (b,x,y,z), device. Sites must be distinct and satisfy
 *          0 <= b < batch, 0 <= x < grid[0], 0 <= y < grid[1], 0 <= z < grid[2].
 * n        number of sites (n = 0 gives an empty map).
 * batch    number of batch items (>= 1).
 * grid     host array of 3 positive extents.
 * flags    0 or SUBMCONV_FLAG_MORTON (iteration order only; results are the
 *          same bit for bit either way), optionally | SUBMCONV_FLAG_SORTED_KEYS
 *          (another lookup structure, the same map) and at most one of
 *          SUBMCONV_FLAG_TILES_256 / SUBMCONV_FLAG_TILES_288.
 * out_map  receives the handle (host pointer).
 *
 * The map is built on `stream`. The function waits for that stream twice:
 * once to read back the validation flags and the active-pair count, when it
 * returns SUBMCONV_ERR_COORD_OUT_OF_RANGE or SUBMCONV_ERR_DUPLICATE_COORD,
 * with no handle, for invalid sites; and once at the end, so that the map
 * is complete on return. The map's device memory is 27*n*4 bytes for the
 * neighbour table plus the per-tile lists (8 bytes per active pair and tile
 * set; a sparse map's wider tiles also keep the order, 4 bytes per tile, in
 * which a forward's workgroups walk them). The build's scratch (the hash table: at least 2n slots of 8 bytes,
 * or 12 when packed keys exceed 32 bits; 8 bytes of key per site; sort space
 * with SUBMCONV_FLAG_MORTON or SUBMCONV_FLAG_SORTED_KEYS) stays with the
 * device after the call, up to 256 MiB, for the next build, until the
 * process ends; so do the four 14 MiB buffers that forwards on W stage the
 * weights in (see submconv_forward), allocated by the first build on the
 * device.
 * Builds on one device run one at a time.
 */
int submconv_build_map(const int32_t* coords, int64_t n, int32_t batch, const int32_t grid[3],
                       uint32_t flags, hipStream_t stream, submconv_map_t* out_map);

/*
 * submconv_release_scratch -- free the build scratch that the current device
 * keeps for its next map build (see submconv_build_map); waits for a build in
 * progress on the device and for the device itself. Maps, prepared weights
 * and the weight stage (4 x 14 MiB) are not affected; the next build allocates its
 * scratch again. Host call, safe at any time.
 */
int submconv_release_scratch(void);

/* Number of sites of the map. */
int64_t submconv_map_num_rows(submconv_map_t map);

/* Rows per tile of the map's widest per-tile neighbour lists: 256 .. 288
 * (see SUBMCONV_FLAG_TILES_256). Negative on a bad argument. */
int32_t submconv_map_tile_rows(submconv_map_t map);

/* Number of (row, tap) pairs with a neighbour, the centre tap included
 * (ksize 3), or n (ksize 1). Effective work of a forward is
 * 2 * active_pairs * Cin * Cout flops. Negative on a bad argument. */
int64_t submconv_map_active_pairs(submconv_map_t map, int32_t ksize);

/* Size of the map's staged plan (see SUBMCONV_FLAG_STAGED): out[0] = units,
 * out[1] = staged rows over all units; both 0 when the map has none. The
 * plan's device memory is 16 bytes per unit, 4 per staged row and 54 per
 * row (n rounded up to even). Returns 0, or a negative status for a NULL
 * argument. */
int submconv_map_staged(submconv_map_t map, int64_t out[2]);

/*
 * submconv_map_export -- write the neighbour map in the caller's row order
 * (the indice map the README's "What's in it" SparseTensor row caches; the
 * naive check of its "Correctness" section compares against the same table).
 * kmap [n,27] int32, device: kmap[i][k] = row j of the site coords[i] + d_k in
 * the same batch item, or -1. Asynchronous on `stream`.
 */
int submconv_map_export(submconv_map_t map, int32_t* kmap, hipStream_t stream);

/*
 * submconv_map_order -- write the internal row processing order:
 * order[t] = caller row processed t-th (identity without the Morton flag).
 * order [n] int32, device. Asynchronous on `stream`.
 */
int submconv_map_order(submconv_map_t map, int32_t* order, hipStream_t stream);

/* Release the map's device memory (waits for the device). NULL is a no-op. */
int submconv_map_free(submconv_map_t map);

/* ------------------------------------------------------------------------
 * Layer weights. W is [K,Cin,Cout] row-major (K = 27 for a 3x3x3 kernel, 1
 * for 1x1x1), 16-bit elements, out = feats @ W[k] per tap k as above. The
 * MFMA kernels read the weights in a fragment order of their own; the calls
 * below that take W rearrange it on the fly (a small kernel on `stream`,
 * into a fixed per-device buffer of the library), and a prepared-weights
 * handle holds the rearranged copy for layers that run many times (the
 * README's "Performance" section caches what it prepares; the forward of
 * the issue #1 thread's "Fixed" list works on the framework's own device
 * tensors).
 * ---------------------------------------------------------------------- */

/* Opaque prepared weights of one layer: library-owned device memory on the
 * device that was current at submconv_weights_create, with the layer's
 * shape, element type and use recorded, so that a forward can check them. */
typedef struct submconv_weights_s* submconv_weights_t;

/*
 * submconv_weights_create -- allocate prepared weights for a layer.
 * ksize 3 or 1; Cin, Cout positive multiples of 8 up to 1024 (the layer's
 * W is [K,Cin,Cout]); dtype SUBMCONV_DTYPE_F16 or SUBMCONV_DTYPE_BF16;
 * flags 0 (for submconv_forward_prepared and submconv_forward_masked) or
 * SUBMCONV_PREP_INPUT_GRAD (for submconv_backward_input_prepared).
 * Allocates K*Cin*Cout*2 bytes on the current device; the content is
 * undefined until submconv_weights_set. *out receives the handle.
 */
int submconv_weights_create(int32_t ksize, int32_t cin, int32_t cout, int32_t dtype,
                            uint32_t flags, submconv_weights_t* out);

/*
 * submconv_weights_set -- prepare the values of W [K,Cin,Cout] (device, the
 * handle's shape and element type, 16-byte aligned) into the handle: W
 * itself, or with SUBMCONV_PREP_INPUT_GRAD the flipped, transposed kernel
 * W_t[k] = W[K-1-k]^T of the input gradient. 16-bit elements are moved
 * without conversion. Asynchronous on `stream`, no allocation; call it again
 * whenever W changes.
 */
int submconv_weights_set(submconv_weights_t w, const uint16_t* W, hipStream_t stream);

/* Release prepared weights (waits for the device). NULL is a no-op. */
int submconv_weights_free(submconv_weights_t w);

/*
 * submconv_forward -- one SubMConv3d layer on the sites of `map` (the
 * operation at the top of this file: the README's "What's in it" SubMConv3d
 * row, computed as the fused product of its "Performance" section).
 *
 * feats  [n,Cin] fp16, device, caller row order.
 * W      [K,Cin,Cout] fp16, device: the layer's weights as they are.
 * bias   [Cout] fp32, device, 16-byte aligned, or NULL for no bias.
 * out    [n,Cout] fp16, device, caller row order; must not overlap feats.
 * ksize  3 (27 taps, uses the neighbour map) or 1 (centre tap only).
 *
 * Accumulates in fp32, adds the bias in fp32 and rounds once to fp16 (round to
 * nearest even). Cin and Cout must be multiples of 8 and at most 1024;
 * feats, W and out 16-byte aligned; map, W's buffer and the current device
 * the same device (SUBMCONV_ERR_INVALID_ARG otherwise).
 * Enqueues on `stream` and does not wait. Every output row is written by
 * exactly one workgroup without atomics, so results are bitwise
 * reproducible run to run, and the same for any row order and tile size.
 *
 * Kernels: Cin in {32, 64, 128} with Cout a multiple of 32, and Cin = 256
 * with Cout a multiple of 128, run the MFMA gather-GEMM; its buffer offsets
 * are 32-bit, so feats ([n,Cin] * 2 bytes) and the map's per-tile lists
 * (8 bytes per active pair) must each stay below 2 GiB, or the call returns
 * SUBMCONV_ERR_UNSUPPORTED_SHAPE before enqueueing anything
 * (submconv_forward_kernel tells which case applies). Other channel counts
 * run a VALU kernel with 64-bit addressing.
 *
 * Allocation: none. For the MFMA kernels W is rearranged first into a
 * staging buffer of the library (14 MiB each, the largest MFMA layer; the
 * first map build on a device allocates four, and they stay until the
 * process ends, like the build's scratch). The first three streams that
 * forward on W on a device each own one buffer, which the stream's own order
 * protects; forwards from any further streams share the fourth and are
 * ordered after one another through an event on it (none is recorded while
 * `stream` is being captured into a graph). A captured forward must not run
 * at the same time as another forward on W from the stream it was captured
 * on, nor, if that stream shares the fourth buffer, from any stream that
 * shares it; a stream handle that is destroyed and created again counts as
 * the same stream. Forwards with prepared weights
 * (submconv_forward_prepared) run concurrently on any streams.
 */
int submconv_forward(submconv_map_t map, const uint16_t* feats, const uint16_t* W,
                     const float* bias, uint16_t* out, int32_t cin, int32_t cout, int32_t ksize,
                     hipStream_t stream);

/*
 * submconv_forward_dtype -- submconv_forward for fp16 (SUBMCONV_DTYPE_F16)
 * or bf16 (SUBMCONV_DTYPE_BF16) features, weights and output (the issue #1
 * thread's "Fixed" list names fp16 and bf16 forwards). Products are
 * accumulated in fp32 (v_mfma_f32_32x32x16_bf16 for bf16), the fp32 bias
 * added, and the result rounded once to the element type (round to nearest
 * even). Otherwise as submconv_forward.
 */
int submconv_forward_dtype(submconv_map_t map, const uint16_t* feats, const uint16_t* W,
                           const float* bias, uint16_t* out, int32_t cin, int32_t cout,
                           int32_t ksize, int32_t dtype, hipStream_t stream);

/*
 * submconv_forward_prepared -- submconv_forward_dtype with weights prepared
 * by submconv_weights_set (created without SUBMCONV_PREP_INPUT_GRAD): ksize,
 * Cin, Cout and the element type are the handle's. Saves the rearrangement
 * (one small kernel) per call and takes no shared buffer: forwards on one
 * map run concurrently on several streams. Asynchronous, no allocation.
 */
int submconv_forward_prepared(submconv_map_t map, const uint16_t* feats, submconv_weights_t w,
                              const float* bias, uint16_t* out, hipStream_t stream);

/*
 * submconv_forward_kernel -- which kernel a forward of this shape takes on a
 * map built with default flags, on the host, without a device: 2 the staged
 * gather-GEMM (a 3x3x3 forward of 32 -> 32, 64 -> 32, 32 -> 64, 128 -> 256
 * or 256 -> 256 channels on a dense map, see SUBMCONV_FLAG_STAGED), 1 the
 * MFMA gather-GEMM on the per-tile lists, 0 the VALU kernel, or a negative
 * status:
 * SUBMCONV_ERR_UNSUPPORTED_SHAPE for an MFMA shape whose features or lists
 * reach 2 GiB (submconv_forward's limit), or a shape error. n rows,
 * active_pairs as submconv_map_active_pairs reports them.
 */
int submconv_forward_kernel(int64_t n, int64_t active_pairs, int32_t cin, int32_t cout,
                            int32_t ksize);

/*
 * submconv_backward_input -- gradient of a layer's loss with respect to its
 * input features (the issue #1 thread's "Fixed" list: "bwd-input").
 *
 * grad_out [n,Cout] fp16, device: dL/dout, caller row order.
 * W        [K,Cin,Cout] fp16, device: the layer's weights as they are.
 * grad_in  [n,Cin] fp16, device: dL/dfeats[j] = sum over (i,k) with
 *          coords[j] = coords[i] + d_k of grad_out[i] @ W[k]^T, accumulated in
 *          fp32 and rounded once (round to nearest even).
 *
 * The terms of row j are the sites i at coords[j] - d_k = coords[j] +
 * d_(K-1-k), so this is the forward on the same map with the flipped,
 * transposed kernel (Cout -> Cin channels, no bias): same requirements,
 * kernels, limits and staging as submconv_forward (with Cin and Cout
 * swapped), asynchronous, no allocation, bitwise reproducible.
 */
int submconv_backward_input(submconv_map_t map, const uint16_t* grad_out, const uint16_t* W,
                            uint16_t* grad_in, int32_t cin, int32_t cout, int32_t ksize,
                            hipStream_t stream);

/* submconv_backward_input for fp16 or bf16 data (SUBMCONV_DTYPE_*). */
int submconv_backward_input_dtype(submconv_map_t map, const uint16_t* grad_out, const uint16_t* W,
                                  uint16_t* grad_in, int32_t cin, int32_t cout, int32_t ksize,
                                  int32_t dtype, hipStream_t stream);

/*
 * submconv_backward_input_prepared -- submconv_backward_input with the
 * layer's weights prepared under SUBMCONV_PREP_INPUT_GRAD (the handle's
 * Cin, Cout, ksize and element type are the layer's). Concurrent on any
 * streams; asynchronous, no allocation.
 */
int submconv_backward_input_prepared(submconv_map_t map, const uint16_t* grad_out,
                                     submconv_weights_t w, uint16_t* grad_in, hipStream_t stream);

/*
 * submconv_backward_weight_workspace_bytes -- device workspace that
 * submconv_backward_weight needs for this map and shape (0 is possible):
 * fp32 partial sums of dW per workgroup. On a map with a staged plan (see
 * SUBMCONV_FLAG_STAGED) a 3x3x3 weight gradient of 32 -> 32, 64 -> 32 or
 * 32 -> 64 channels works per staged unit, with partials of all 27 taps per
 * workgroup (about 54 MiB at 64 -> 32 on 256 compute units). Negative on a
 * bad argument.
 */
int64_t submconv_backward_weight_workspace_bytes(submconv_map_t map, int32_t cin, int32_t cout,
                                                 int32_t ksize);

/*
 * submconv_backward_weight -- gradient of a layer's loss with respect to its
 * weights (the issue #1 thread's "bwd-weight").
 *
 * feats     [n,Cin] fp16, device: the layer's input, caller row order.
 * grad_out  [n,Cout] fp16, device: dL/dout, caller row order.
 * grad_w    [K,Cin,Cout] fp32, device, overwritten: dL/dW[k] = sum over the
 *           rows i with a neighbour j at coords[i] + d_k of
 *           feats[j]^T grad_out[i] (outer products), fp32 accumulation.
 * workspace device buffer of submconv_backward_weight_workspace_bytes bytes
 *           (may be NULL when that is 0); its content is scratch.
 *
 * Enqueues on `stream`, allocates nothing and does not wait. Partial sums
 * are combined in a fixed order, so results are bitwise reproducible.
 * Cin and Cout must be multiples of 8 and at most 1024. feats, grad_out,
 * grad_w and workspace must be 16-byte aligned (SUBMCONV_ERR_INVALID_ARG
 * otherwise).
 */
int submconv_backward_weight(submconv_map_t map, const uint16_t* feats, const uint16_t* grad_out,
                             float* grad_w, void* workspace, int32_t cin, int32_t cout,
                             int32_t ksize, hipStream_t stream);

/*
 * submconv_backward_weight_noalloc -- submconv_backward_weight for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same kernels, with the
 * partial sums in a fixed 32 MiB workspace that is part of the library's
 * device code (one per device, held until the process ends) instead of a
 * caller's workspace. When the partials of the allocating entry point's work
 * split would not fit, workgroups take longer runs of tiles (down to one run
 * per tap), so every shape fits; the sum order then differs from
 * submconv_backward_weight's (the same tolerance, not the same bits).
 * Arguments, requirements and results as submconv_backward_weight. The call
 * never allocates, frees or calls an allocating library routine. All calls on
 * one device share its workspace, which keeps the last call's contents: calls
 * that overlap in time on one device (several streams or threads) race and
 * must be ordered by the caller. Asynchronous on `stream`.
 */
int submconv_backward_weight_noalloc(submconv_map_t map, const uint16_t* feats,
                                     const uint16_t* grad_out, float* grad_w, int32_t cin,
                                     int32_t cout, int32_t ksize, hipStream_t stream);

/*
 * submconv_backward_bias -- gradient with respect to the bias: grad_b[c] =
 * sum over the n rows of grad_out[row][c] (fp16 in, fp32 accumulation and
 * result), summed in a fixed order (bitwise reproducible). grad_out [n,Cout]
 * fp16 and grad_b [Cout] fp32, device; Cout a multiple of 8 up to 1024.
 * Asynchronous on `stream`, no allocation.
 */
int submconv_backward_bias(const uint16_t* grad_out, int64_t n, int32_t cout, float* grad_b,
                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * Masked implicit-GEMM forward: the variant the trellis-mac issue #1 thread
 * measures against its dense kernel ("Fixed" list and the dense-vs-masked
 * table). Rows are sorted by their 27-bit neighbour mask (sorted_idx); each
 * block of 64 sorted rows runs the taps in the union of its rows' masks
 * (valid_kernel / valid_kernel_seg), every row taking part with zeros where
 * its neighbour is absent. Same result as submconv_forward (fp32
 * accumulation, one rounding), different cost: fp32 accumulators in
 * registers, but each tap padded to the block.
 * ---------------------------------------------------------------------- */

typedef struct submconv_masked_s* submconv_masked_t;

/*
 * submconv_masked_plan -- sort the map's rows by neighbour mask and build the
 * per-block tap lists and neighbour tables (about 4 bytes per (block row, run
 * tap)). Builds on `stream` and waits for it twice; makes two device
 * allocations, held until submconv_masked_free: the block arrays with the
 * build's temporaries (about 28 bytes per row, plus the radix sort's scratch),
 * then the tap lists and neighbour tables. The plan refers to `map`'s buffers:
 * free it before the map.
 */
int submconv_masked_plan(submconv_map_t map, hipStream_t stream, submconv_masked_t* out_plan);

/* (row, tap) products the masked forward executes, padding included
 * (64 x the number of block taps); negative on a bad argument. */
int64_t submconv_masked_row_taps(submconv_masked_t plan);

/*
 * submconv_forward_masked -- the masked forward of a 3x3x3 layer: arguments as
 * submconv_forward_prepared, with fp16 weights prepared for (3, Cin, Cout)
 * (no SUBMCONV_PREP_INPUT_GRAD); Cin in {32, 64, 128} with Cout a multiple of
 * 32, or Cin 256 with Cout a multiple of 128; features below 2 GiB.
 * Asynchronous, no allocation, bitwise reproducible.
 */
int submconv_forward_masked(submconv_masked_t plan, const uint16_t* feats, submconv_weights_t w,
                            const float* bias, uint16_t* out, hipStream_t stream);

/* Release a masked plan (waits for the device). NULL is a no-op. */
int submconv_masked_free(submconv_masked_t plan);

/* ------------------------------------------------------------------------
 * Coordinate operations of the same sparse stack (trellis_sparse_mlx README,
 * "What's in it" table, subdivide / downsample row): x2 max-pooling and x2
 * coordinate expansion.
 * ---------------------------------------------------------------------- */

/* Opaque downsample plan: library-owned device buffers describing which
 * sites fall into which parent; immutable, released by submconv_downsample_free. */
typedef struct submconv_down_s* submconv_down_t;

/*
 * submconv_downsample_plan -- group the sites by parent (b, x/2, y/2, z/2).
 *
 * coords [n,4] int32 (b,x,y,z), device, 0 <= b < batch, 0 <= x < grid[0],
 * ... (a repeated site is simply one more child). The parents are the
 * distinct parent sites in ascending lexicographic (b,x,y,z) order; the
 * parent grid is ceil(grid/2). Builds on `stream`, then waits for it once (to
 * learn the parent count and report SUBMCONV_ERR_COORD_OUT_OF_RANGE). Makes one
 * device allocation, held until submconv_downsample_free: the plan's arrays (28
 * bytes per site) and the build's temporaries (16 bytes per site, 24 when
 * batch * ceil(grid/2) products exceed 2^32, plus the radix sort's scratch).
 */
int submconv_downsample_plan(const int32_t* coords, int64_t n, int32_t batch, const int32_t grid[3],
                             hipStream_t stream, submconv_down_t* out_plan);

/* Number of parents M of a plan (negative on a bad argument). */
int64_t submconv_downsample_rows(submconv_down_t plan);

/* Parent grid extents (host array of 3). */
int submconv_downsample_grid(submconv_down_t plan, int32_t pgrid[3]);

/*
 * submconv_downsample_coords -- pcoords [M,4] int32 (parent sites, sorted) and
 * inverse [n] int32 (parent row of each site); either may be NULL. Device
 * pointers, asynchronous on `stream`.
 */
int submconv_downsample_coords(submconv_down_t plan, int32_t* pcoords, int32_t* inverse,
                               hipStream_t stream);

/*
 * submconv_downsample_max -- parent features: out[p][c] = max over the sites
 * of parent p of feats[site][c] (fp16, exact). feats [n,C] and out [M,C] fp16,
 * device, 16-byte aligned, C a multiple of 8 up to 4096. Asynchronous, no
 * allocation; may be called for any number of feature tensors per plan.
 */
int submconv_downsample_max(submconv_down_t plan, const uint16_t* feats, int32_t cdim, uint16_t* out,
                            hipStream_t stream);

/* Release a plan (waits for the device). NULL is a no-op. */
int submconv_downsample_free(submconv_down_t plan);

/*
 * submconv_subdivide -- x2 expansion: site i becomes the rows 8i + c,
 * c = 4dx + 2dy + dz (dx slowest), at (b, 2x+dx, 2y+dy, 2z+dz), each with site
 * i's feature row. coords [n,4] int32, out_coords [8n,4] int32; feats [n,C]
 * and out_feats [8n,C] fp16 (both NULL for coordinates only; C a multiple of
 * 8 up to 4096, 16-byte aligned). Device pointers, asynchronous, no allocation.
 */
int submconv_subdivide(const int32_t* coords, int64_t n, const uint16_t* feats, int32_t cdim,
                       int32_t* out_coords, uint16_t* out_feats, hipStream_t stream);

/* Message for a status code (static string). */
const char* submconv_status_string(int status);

/* Thread-local detail message of the last failing call on this thread. */
const char* submconv_last_error(void);

/* SUBMCONV_ABI_VERSION of the built library. */
int submconv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SUBMCONV_H_ */
