/*
 * submconv.h -- C ABI of the MI355X (gfx950) submanifold 3x3x3 sparse
 * convolution library (SubMConv3d).
 *
 * The operation (lato.2_mrp_mlx working notes, commit summary and section
 * "Key facts"): a sparse tensor is a set of N active voxels with integer
 * coordinates (b, z, y, x) and a feature row each.  The submanifold
 * convolution keeps the output set equal to the input set (stride 1, no
 * dilation of the set) and computes, for every active voxel i,
 *
 *     out[i] = bias + sum over the 27 offsets d in {-1,0,1}^3 of W[d] . feats[j]
 *
 * where j is the active voxel at coords[i] + d in the same batch entry (taps
 * with no active voxel there contribute nothing).  Weights use the KRSC layout
 * [Cout, kz, ky, kx, Cin] of the upstream sparse library.  The neighbour lookup
 * is done once per coordinate set and reused by every convolution on that set
 * (same page, commit summary: a map cached per coordinate set).
 *
 * Conventions fixed here where the pages are silent:
 *   - tap k <-> offset (dz, dy, dx) = (k/9 - 1, (k/3)%3 - 1, k%3 - 1), i.e. C
 *     order over the kernel's (kz, ky, kx); kernel axis a pairs with coordinate
 *     column a+1; k = 13 is the centre.
 *   - orientation: correlation by default (the neighbour at c + d is weighted by
 *     W[kz,ky,kx] with (kz,ky,kx) = d + 1); flip = 1 selects the mirrored kernel,
 *     W at 1 - d (the pages leave the orientation open, "Unresolved" section).
 *   - neighbours outside [0, res)^3 or in another batch entry do not exist.
 *
 * Memory: every tensor pointer is a DEVICE pointer owned by the caller unless
 * stated otherwise; rows are contiguous, row-major.  A rulebook and its device
 * memory are owned by the library from submconv_build_map until
 * submconv_rulebook_free.
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = null stream).  All
 * work is enqueued on it.  Only calls that must return a device-computed value
 * (build_map's validity status, output row counts) wait for that stream's work.
 *
 * Errors: every call returns a status (0 = success, < 0 = error); no call aborts
 * or throws.  Host-side argument checks run before any HIP call.
 * submconv_status_string names a status; submconv_last_error gives the detail
 * of the last failure on the calling thread.
 */
#ifndef SUBMCONV_H
#define SUBMCONV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SUBMCONV_OK 0
#define SUBMCONV_E_INVALID_ARG (-1) /* null pointer, bad size, misaligned pointer, ... */
#define SUBMCONV_E_COORD_RANGE (-2) /* a coordinate outside [0,res) or batch outside [0,batch) */
#define SUBMCONV_E_DUPLICATE (-3)   /* two rows with the same (b, z, y, x) */
#define SUBMCONV_E_UNSUPPORTED (-4) /* channel count / dtype / grid size not supported */
#define SUBMCONV_E_ALIAS (-5)       /* an output buffer overlaps an input buffer */
#define SUBMCONV_E_OOM (-6)         /* device allocation failed */
#define SUBMCONV_E_HIP (-7)         /* a HIP runtime call or kernel launch failed */

/* Element types of feature, weight and output tensors (bias is always fp32). */
#define SUBMCONV_F32 0
#define SUBMCONV_BF16 1

/* Forward kernel selection (submconv_forward_variant). */
#define SUBMCONV_KERNEL_AUTO 0    /* pick by (Cin, Cout, dtype, N) */
#define SUBMCONV_KERNEL_GENERIC 1 /* one thread per output element, any channel counts */
#define SUBMCONV_KERNEL_LOWC 2    /* narrow channels (<= 32), wave shuffles, no matrix cores */
#define SUBMCONV_KERNEL_MFMA 3    /* implicit GEMM on matrix cores, Cin/Cout in {32,64,128}, or 16 -> 16 */
#define SUBMCONV_KERNEL_WINDOW 4  /* matrix cores fed from a tile's neighbourhood staged in LDS
                                     (bf16, Cin = Cout = 32, N * 64 <= 2^31 - 1; otherwise
                                     SUBMCONV_E_UNSUPPORTED) */
#define SUBMCONV_KERNEL_PERSISTENT 5 /* persistent matrix-core kernel, weights streamed through LDS,
                                        operands gathered into registers (bf16, 64->64 or 128->128,
                                        N * Cin * 2 <= 2^31 - 1; otherwise SUBMCONV_E_UNSUPPORTED) */

typedef struct submconv_rulebook submconv_rulebook; /* opaque, library-owned */

/*
 * Build the neighbour map ("rulebook") of a coordinate set.
 *
 *   coords : device int32 [n,4], rows (b, z, y, x), 16-byte aligned; any row order.
 *   n      : number of rows, 0 <= n < 2^31 (n = 0 gives an empty rulebook).
 *   res    : grid extent per spatial axis (cubic grid), 1 <= res.
 *   batch  : number of batch entries; every b must satisfy 0 <= b < batch.
 *            (3 * bits(res-1) + bits(batch-1) must not exceed 64.)
 *   stream : hipStream_t.
 *   out_rb : receives the rulebook on success, NULL on failure.
 *
 * The table computed is nbr int32 [n,27]: nbr[i,k] = row of the voxel at
 * coords[i] + offset(k), or -1.  It is exact (integer work).  It waits for the
 * build to finish to learn the validity status: E_COORD_RANGE if a coordinate is
 * out of range, E_DUPLICATE if two rows are equal (no rulebook is returned).  On
 * the bitmap path (grids of at most 2^31 keys) and for sets of at most 2048 voxels,
 * the build's last kernel writes the status to pinned host memory and the call polls
 * it instead of synchronising the stream (for at most ~2 ms, then it synchronises);
 * when it returns, the rulebook's contents are complete, though the stream may not
 * yet be idle.
 * Device memory comes from the library's block cache (submconv_release_cache),
 * else from the device's stream-ordered pool.
 *
 * `batch` is an argument the pages' interface does not have: it bounds the batch
 * index so the key width is known on the host without reading the coordinates
 * back (one synchronisation fewer).
 */
int submconv_build_map(const int32_t *coords, int64_t n, int32_t res, int32_t batch,
                       void *stream, submconv_rulebook **out_rb);

/* Device pointer to the nbr table int32 [n,27] in input row order (owned by the
 * rulebook, valid until it is freed) and its row count.  The rulebook keeps its
 * table by sorted position; the input-order copy is built on the first call, on
 * `stream` (one allocation and one kernel), and reused afterwards. */
int submconv_rulebook_neighbors(submconv_rulebook *rb, void *stream, const int32_t **nbr, int64_t *n);

/* Write the nbr table int32 [n,27] in input row order into caller memory dst
 * (device), enqueued on `stream`. */
int submconv_rulebook_copy_neighbors(const submconv_rulebook *rb, int32_t *dst, void *stream);

/* Host-side facts of a rulebook: rows, grid, batch count, and P = number of
 * entries of nbr that are not -1 (centre taps included). */
int submconv_rulebook_info(const submconv_rulebook *rb, int64_t *n, int32_t *res, int32_t *batch,
                           int64_t *taps_present);

/* Release a rulebook; its memory returns to the pool in order on `stream`
 * (work already queued on other streams that uses it must be ordered first).
 * NULL is accepted. */
int submconv_rulebook_free(submconv_rulebook *rb, void *stream);

/*
 * Submanifold convolution forward pass on a rulebook's coordinate set.
 *
 *   feats  : device [n, cin] of dtype, row i = voxel of coords row i.
 *   weight : device KRSC [cout, 3, 3, 3, cin] of dtype.
 *   bias   : device fp32 [cout], or NULL for none (added once).
 *   out    : device [n, cout] of dtype; must not overlap feats or weight (E_ALIAS).
 *   cin, cout : 1..1024; the matrix-core path takes {32, 64, 128} x {32, 64, 128}
 *            and 16 -> 16, the rest runs on the generic kernels.
 *   dtype  : SUBMCONV_F32 or SUBMCONV_BF16; accumulation is fp32, bf16 output is
 *            one round-to-nearest-even of the fp32 sum.
 *   flip   : 0 = correlation, 1 = mirrored kernel (weight tap 26 - k for tap k).
 *
 * Pointers must be aligned to 16 bytes.  Asynchronous: never synchronises,
 * allocates nothing and clears no memory; it is one kernel launch on `stream`, so a
 * caller may capture it in a HIP graph and replay it (the rulebook, the buffers and
 * the weights must then stay allocated, and a replay reads their current contents).
 */
int submconv_forward(const void *feats, const void *weight, const float *bias,
                     const submconv_rulebook *rb, void *out, int32_t cin, int32_t cout,
                     int32_t dtype, int32_t flip, void *stream);

/* submconv_forward with an explicit kernel choice (SUBMCONV_KERNEL_*), for
 * A/B measurement; E_UNSUPPORTED if that kernel does not take these sizes. */
int submconv_forward_variant(const void *feats, const void *weight, const float *bias,
                             const submconv_rulebook *rb, void *out, int32_t cin, int32_t cout,
                             int32_t dtype, int32_t flip, int32_t variant, void *stream);

/*
 * Subdivide (lato.2_mrp_mlx working notes, "Key facts": upsampling is
 * coords*2 + unit cube with features replicated): parent i -> children
 * 8i + q, q = 4 dz + 2 dy + dx (C order), coords (b, 2z+dz, 2y+dy, 2x+dx),
 * feats row copied.  coords device int32 [n,4] with 0 <= z,y,x < 2^30;
 * feats [n,c] of dtype or NULL (then out_feats is ignored);
 * out_coords [8n,4]; out_feats [8n,c].  Asynchronous.
 */
int submconv_subdivide(const int32_t *coords, const void *feats, int64_t n, int32_t c,
                       int32_t dtype, int32_t *out_coords, void *out_feats, void *stream);

/*
 * Sparse space-to-depth with factor 2 (trellis_sparse_mrp_mlx commits, the
 * spatial2channel commit): each fine voxel goes to coarse voxel
 * (b, z/2, y/2, x/2), slot s = (z%2) + 2 (y%2) + 4 (x%2) (axis 0 fastest).
 *
 *   coords [n,4], feats [n,c]: fine set, validated like submconv_build_map
 *            against res and batch (E_COORD_RANGE, E_DUPLICATE).
 *   out_coords : [capacity >= n, 4] -> coarse coords, ascending (b, z, y, x).
 *   out_feats  : [capacity >= n, 8c] -> slot s at channels [s c, (s+1) c);
 *            slots with no fine voxel are zero.
 *   out_mask   : uint8 [capacity >= n, 8] -> 1 where the slot is occupied; may be NULL.
 *   out_m      : host int64, receives M, the number of coarse voxels.
 * Synchronises `stream` to read M and the status.
 */
int submconv_space_to_depth(const int32_t *coords, const void *feats, int64_t n, int32_t c,
                            int32_t dtype, int32_t res, int32_t batch, int32_t *out_coords,
                            void *out_feats, uint8_t *out_mask, int64_t *out_m, void *stream);

/*
 * Inverse of submconv_space_to_depth: coarse voxel m emits child slot s
 * (s ascending; child (b, 2z + s%2, 2y + (s/2)%2, 2x + s/4)) with features
 * coarse_feats[m, s c : (s+1) c] -- every slot when mask is NULL, else only the
 * slots with mask[m,s] != 0 (the masked channel2spatial of the same commit).
 *   coarse_coords [m,4], coarse_feats [m, 8c], mask uint8 [m,8] or NULL,
 *   out_coords [capacity >= 8m, 4], out_feats [capacity >= 8m, c],
 *   out_n : host int64, receives the number of children written.
 * With a mask it synchronises `stream` to read the count; without, it does not.
 */
int submconv_depth_to_space(const int32_t *coarse_coords, const void *coarse_feats,
                            const uint8_t *mask, int64_t m, int32_t c, int32_t dtype,
                            int32_t *out_coords, void *out_feats, int64_t *out_n, void *stream);

/*
 * Masked upsample (trellis_sparse_mrp_mlx commits, the commit closing the op gap
 * for Pixal3D: a masked expansion, distinct from subdivide): voxel i emits child
 * slot s iff mask[i, s] != 0, s ascending, child (b, 2z + s%2, 2y + (s/2)%2,
 * 2x + s/4) -- axis 0 fastest, the reverse of subdivide's C order -- whose
 * feature row is a copy of feats[i].  A voxel with no flagged slot emits nothing.
 *   coords device int32 [n,4] (0 <= z,y,x < 2^30), feats device [n,c] of dtype,
 *   mask device uint8 [n,8]; out_coords [capacity >= 8n, 4], out_feats
 *   [capacity >= 8n, c]; out_n host int64, receives the number of children
 *   (children of voxel i follow those of voxel i-1).
 * Synchronises `stream` once to read the count.  Outputs must not overlap inputs
 * (E_ALIAS).
 */
int submconv_upsample_masked(const int32_t *coords, const void *feats, const uint8_t *mask, int64_t n, int32_t c,
                             int32_t dtype, int32_t *out_coords, void *out_feats, int64_t *out_n, void *stream);

/*
 * submconv_upsample_masked for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, results and errors as submconv_upsample_masked, and the same kernels, but
 * the scratch (per-voxel child counts, their scan, the total) lives in one fixed device
 * array of SUBMCONV_NOALLOC_SCRATCH_BYTES per GPU, which the library holds from the
 * first call on that GPU until the process ends.  The call makes no hipMalloc, hipFree
 * or other allocating call; the child count is read back through a host stack word.
 *
 *   n : 0 <= n <= SUBMCONV_NOALLOC_MAX_N, else E_UNSUPPORTED (checked before any
 *       device work).
 *
 * Every call on a GPU uses that GPU's one array; nothing in it needs clearing (each
 * word read is written first by the same call).  Calls that overlap in time on one GPU
 * (from several host threads or on several streams) race on the array and must be
 * serialised by the caller.  Synchronises `stream` once to read the count.
 */
#define SUBMCONV_NOALLOC_SCRATCH_BYTES (32u << 20)
#define SUBMCONV_NOALLOC_MAX_N 4000000
int submconv_upsample_masked_noalloc(const int32_t *coords, const void *feats, const uint8_t *mask, int64_t n,
                                     int32_t c, int32_t dtype, int32_t *out_coords, void *out_feats,
                                     int64_t *out_n, void *stream);

/* Pooling modes of submconv_downsample. */
#define SUBMCONV_POOL_MAX 0
#define SUBMCONV_POOL_MEAN 1

/*
 * Sparse downsample by 2 (same commit: the mode differs between models and must be
 * explicit): every coarse voxel (b, z/2, y/2, x/2) that holds a fine voxel gets the
 * channel-wise maximum (SUBMCONV_POOL_MAX, exact) or mean (SUBMCONV_POOL_MEAN: fp32
 * sum over its occupied children in slot order, divided by their count, one rounding
 * to the output type) of its children's feature rows.
 *   coords [n,4], feats [n,c]: fine set, validated like submconv_build_map against
 *            res and batch (E_COORD_RANGE, E_DUPLICATE).
 *   out_coords : [capacity >= n, 4] -> coarse coords, ascending (b, z, y, x).
 *   out_feats  : [capacity >= n, c] -> pooled rows.
 *   out_m      : host int64, receives M, the number of coarse voxels.
 * Synchronises `stream` to read M and the status.
 */
int submconv_downsample(const int32_t *coords, const void *feats, int64_t n, int32_t c, int32_t dtype, int32_t res,
                        int32_t batch, int32_t mode, int32_t *out_coords, void *out_feats, int64_t *out_m,
                        void *stream);

/* Weight layouts of a 3x3x3 kernel. */
#define SUBMCONV_LAYOUT_UNKNOWN (-1)
#define SUBMCONV_LAYOUT_KRSC 0  /* [Cout, kz, ky, kx, Cin] (spconv; what the forward takes) */
#define SUBMCONV_LAYOUT_OIDHW 1 /* [Cout, Cin, kz, ky, kx] (torch Conv3d) */

/*
 * Which layout a 5-D weight shape is (lato.2_mrp_mlx working notes, "Key facts": both
 * layouts are 5-D, so the rank decides nothing).  Host only, no device work.
 *   shape  : host int64 [5].
 *   hint   : SUBMCONV_LAYOUT_UNKNOWN, or the layout the caller's module implies
 *            (a sparse conv module: KRSC; a dense nn.Conv3d: OIDHW).
 *   layout : host, receives SUBMCONV_LAYOUT_KRSC or SUBMCONV_LAYOUT_OIDHW.
 * E_UNSUPPORTED when neither reading is a 3x3x3 kernel; E_INVALID_ARG when the shape
 * fits both ([O,3,3,3,3]) and no hint is given, or the hint contradicts the shape.
 */
int submconv_classify_5d(const int64_t *shape, int32_t hint, int32_t *layout);

/*
 * KRSC weights from either layout, optionally mirrored (flip != 0: tap k of dst is
 * tap 26 - k of src, the kernel the forward's flip option stands for; same page,
 * "Unresolved").  src device [cout,3,3,3,cin] (KRSC) or [cout,cin,3,3,3] (OIDHW) of
 * dtype; dst device KRSC [cout,3,3,3,cin], must not overlap src (E_ALIAS).
 * Asynchronous on `stream`.
 */
int submconv_weight_convert(const void *src, int32_t layout, int32_t cout, int32_t cin, int32_t dtype, int32_t flip,
                            void *dst, void *stream);

/*
 * The library keeps device blocks it has freed (rulebooks, scratch) for reuse on the
 * same device, up to a limit per device (2 GiB unless set below), so that repeated
 * builds make no driver allocation calls.  A block freed while work queued on its
 * stream may still read it carries an event recorded at the free; the next user's
 * stream waits for that event before the block is reused, on any stream.
 *
 * submconv_release_cache returns the cached blocks of `device` (all devices when
 * device < 0) to the driver after their last use has finished.  Blocks in use are not
 * affected.
 */
int submconv_release_cache(int32_t device);

/* Set the per-device limit of the block cache in bytes (0 disables caching); cached
 * blocks beyond the new limit are released.  E_INVALID_ARG if bytes < 0. */
int submconv_set_cache_limit(int64_t bytes);

/* Name of a status code (static string). */
const char *submconv_status_string(int status);

/* Detail of the last failing call on this thread (static thread-local string). */
const char *submconv_last_error(void);

/* Library version string. */
const char *submconv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SUBMCONV_H */
