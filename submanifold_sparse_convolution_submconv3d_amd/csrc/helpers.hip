// Sparse-tensor helpers that produce new coordinate sets.
//
// subdivide       - every voxel becomes its 2x2x2 children in C order, features
//                   replicated (lato.2_mrp_mlx working notes, "Key facts").
// space_to_depth  - factor 2: fine voxel -> coarse voxel (b, z/2, y/2, x/2),
//                   slot (z%2) + 2(y%2) + 4(x%2), axis 0 fastest, features in
//                   channels [slot C, (slot+1) C), empty slots zero
//                   (trellis_sparse_mrp_mlx commits, spatial2channel commit).
//                   Built on the same key packing and radix sort as the map:
//                   the sort key is (coarse key << 3) | slot, so sorted order
//                   groups each coarse voxel's children and exposes duplicates.
// depth_to_space  - inverse: slot s of coarse voxel m -> child s, all slots or
//                   only the masked ones (the masked channel2spatial).
// upsample_masked - voxel i emits child s (decoded like the slots above) iff
//                   mask[i, s] != 0, the child copying the parent's feature row
//                   (trellis_sparse_mrp_mlx commits, the commit closing the op
//                   gap for Pixal3D: masked expansion, distinct from subdivide).
// downsample      - pools each coarse voxel's children by max or mean, coarse
//                   rows ascending (same commit: the mode is explicit); the same
//                   sort as space_to_depth groups the children.
#include <mutex>

#include "common.h"
#include "mailbox.h"

namespace sc {

// ---------------------------------------------------------------------------
// subdivide
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_subdivide_coords(const int4 *__restrict__ in, int64_t n,
                                                          int4 *__restrict__ out)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= 8 * n) return;
    const int64_t i = e >> 3;
    const int q = (int)(e & 7);
    const int4 c = in[i];
    out[e] = make_int4(c.x, 2 * c.y + (q >> 2), 2 * c.z + ((q >> 1) & 1), 2 * c.w + (q & 1));
}

// Row and unit of a flat thread index with `per` units per row (per > 0, a kernel
// argument, so the test is uniform): a shift when per is a power of two, else a
// division, 32-bit while the index fits.  A 64-bit division by a runtime value costs
// more than the 16-byte move these streaming kernels do per thread.
__device__ __forceinline__ int64_t split_index(int64_t e, int per, int &u)
{
    if ((per & (per - 1)) == 0) {
        u = (int)(e & (per - 1));
        return e >> __builtin_ctz((unsigned)per);
    }
    if ((uint64_t)e <= 0xFFFFFFFFull) {
        const uint32_t q = (uint32_t)e / (uint32_t)per;
        u = (int)((uint32_t)e - q * (uint32_t)per);
        return (int64_t)q;
    }
    const int64_t q = e / per;
    u = (int)(e - q * per);
    return q;
}

// Copy each parent row to its 8 children in units V (16-byte vectors or 4-byte words;
// rows are whole units).
template <typename V>
__global__ __launch_bounds__(256) void k_subdivide_feats(const V *__restrict__ in, int64_t n, int words,
                                                         V *__restrict__ out)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over 8n rows x words
    if (e >= 8 * n * words) return;
    int wi;
    const int64_t child = split_index(e, words, wi);
    out[e] = in[(child >> 3) * words + wi];
}

// 2-byte rows that are not whole words (odd bf16 channel counts)
__global__ __launch_bounds__(256) void k_subdivide_feats16(const uint16_t *__restrict__ in,
                                                           int64_t n, int c,
                                                           uint16_t *__restrict__ out)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= 8 * n * c) return;
    int ci;
    const int64_t child = split_index(e, c, ci);
    out[e] = in[(child >> 3) * c + ci];
}

int subdivide(const int32_t *coords, const void *feats, int64_t n, int c, int dtype,
              int32_t *out_coords, void *out_feats, hipStream_t s)
{
    if (n == 0) return SUBMCONV_OK;
    const int64_t kids = 8 * n;
    hipLaunchKernelGGL(k_subdivide_coords, dim3((unsigned)((kids + 255) / 256)), dim3(256), 0, s,
                       (const int4 *)coords, n, (int4 *)out_coords);
    SC_LAUNCHED("subdivide_coords");
    if (feats) {
        const int64_t row_bytes = (int64_t)c * (dtype == SUBMCONV_F32 ? 4 : 2);
        if (row_bytes % 16 == 0 && ((uintptr_t)feats & 15) == 0 && ((uintptr_t)out_feats & 15) == 0) {
            const int vecs = (int)(row_bytes / 16);
            const int64_t total = kids * vecs;
            hipLaunchKernelGGL(k_subdivide_feats<uint4>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                               s, (const uint4 *)feats, n, vecs, (uint4 *)out_feats);
        } else if (row_bytes % 4 == 0) {
            const int words = (int)(row_bytes / 4);
            const int64_t total = kids * words;
            hipLaunchKernelGGL(k_subdivide_feats<uint32_t>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                               s, (const uint32_t *)feats, n, words, (uint32_t *)out_feats);
        } else {
            const int64_t total = kids * c;
            hipLaunchKernelGGL(k_subdivide_feats16, dim3((unsigned)((total + 255) / 256)), dim3(256),
                               0, s, (const uint16_t *)feats, n, c, (uint16_t *)out_feats);
        }
        SC_LAUNCHED("subdivide_feats");
    }
    return SUBMCONV_OK;
}

// ---------------------------------------------------------------------------
// space_to_depth
// ---------------------------------------------------------------------------

template <typename K>
__global__ __launch_bounds__(256) void k_s2d_pack(const int4 *__restrict__ coords, int64_t n,
                                                  int res, int batch, int rbc, K *__restrict__ keys,
                                                  int32_t *__restrict__ rows, DevStatus *st)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int4 c = coords[i];
    const bool bad = (unsigned)c.x >= (unsigned)batch || (unsigned)c.y >= (unsigned)res ||
                     (unsigned)c.z >= (unsigned)res || (unsigned)c.w >= (unsigned)res;
    K key = K(0);
    if (!bad) {
        const K coarse = ((((K)c.x << rbc | (K)(c.y >> 1)) << rbc | (K)(c.z >> 1)) << rbc) | (K)(c.w >> 1);
        const K slot = (K)((c.y & 1) | ((c.z & 1) << 1) | ((c.w & 1) << 2));
        key = (coarse << 3) | slot;
    }
    keys[i] = key;
    rows[i] = (int32_t)i;
    if (bad) atomicOr(&st->flags, FLAG_RANGE);
}

// head[s] = 1 where a new coarse voxel starts in sorted order; duplicates flagged.
template <typename K>
__global__ __launch_bounds__(256) void k_s2d_heads(const K *__restrict__ sk, int64_t n,
                                                   uint32_t *__restrict__ head, DevStatus *st)
{
    const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (s >= n) return;
    const K key = sk[s];
    uint32_t h = 1;
    if (s > 0) {
        const K prev = sk[s - 1];
        h = (prev >> 3) != (key >> 3);
        if (prev == key) atomicOr(&st->flags, FLAG_DUPLICATE);
    }
    head[s] = h;
}

// Zero the coarse rows and write their coordinates (one thread per sorted head).
template <typename K, typename T>
__global__ __launch_bounds__(256) void k_s2d_rows(const K *__restrict__ sk,
                                                  const uint32_t *__restrict__ head,
                                                  const uint32_t *__restrict__ seg, int64_t n,
                                                  int rbc, int c, int4 *__restrict__ out_coords,
                                                  T *__restrict__ out_feats,
                                                  uint8_t *__restrict__ out_mask)
{
    const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (s >= n || !head[s]) return;
    const int64_t m = seg[s];
    if (m >= n) return;
    const K coarse = sk[s] >> 3;
    const K msk = (K(1) << rbc) - 1;
    out_coords[m] = make_int4((int)(coarse >> (3 * rbc)), (int)((coarse >> (2 * rbc)) & msk),
                              (int)((coarse >> rbc) & msk), (int)(coarse & msk));
    T *row = out_feats + m * 8 * c;
    for (int e = 0; e < 8 * c; ++e) row[e] = T(0);
    if (out_mask)
        for (int q = 0; q < 8; ++q) out_mask[m * 8 + q] = 0;
}

// Scatter each fine row into its coarse row's slot (one thread per element).
template <typename K, typename T>
__global__ __launch_bounds__(256) void k_s2d_scatter(const K *__restrict__ sk,
                                                     const int32_t *__restrict__ perm,
                                                     const uint32_t *__restrict__ seg, int64_t n,
                                                     int c, const T *__restrict__ feats,
                                                     T *__restrict__ out_feats,
                                                     uint8_t *__restrict__ out_mask)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= n * c) return;
    int ci;
    const int64_t s = split_index(e, c, ci);
    const int slot = (int)(sk[s] & 7);
    const int64_t m = seg[s];
    const uint32_t src = (uint32_t)perm[s];
    if (m >= n || src >= (uint64_t)n) return;
    out_feats[(m * 8 + slot) * c + ci] = feats[(int64_t)src * c + ci];
    if (ci == 0 && out_mask) out_mask[m * 8 + slot] = 1;
}

// seg[s] = (number of heads at or before s) - 1, from the exclusive scan of head.
__global__ __launch_bounds__(256) void k_excl_to_seg(const uint32_t *__restrict__ head,
                                                     uint32_t *__restrict__ seg, int64_t n)
{
    const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (s < n) seg[s] = seg[s] + head[s] - 1;
}

// A helper call's status to the host's mailbox: the flags its kernels set in `st` (none
// when st is null) and the output row count in *total.
__global__ void k_post_count(const uint32_t *__restrict__ total, const DevStatus *st, Mailbox *mb, uint32_t seq)
{
    mailbox_post(mb, seq, st ? st->flags : 0u, 0ull, (unsigned long long)*total);
}

// Coarse coordinates and the sorted position where each coarse voxel's children start.
template <typename K>
__global__ __launch_bounds__(256) void k_down_rows(const K *__restrict__ sk, const uint32_t *__restrict__ head,
                                                   const uint32_t *__restrict__ seg, int64_t n, int rbc,
                                                   int4 *__restrict__ out_coords, uint32_t *__restrict__ start)
{
    const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (s >= n || !head[s]) return;
    const int64_t m = seg[s];
    if (m >= n) return;
    const K coarse = sk[s] >> 3;
    const K msk = (K(1) << rbc) - 1;
    out_coords[m] = make_int4((int)(coarse >> (3 * rbc)), (int)((coarse >> (2 * rbc)) & msk),
                              (int)((coarse >> rbc) & msk), (int)(coarse & msk));
    start[m] = (uint32_t)s;
}

// Kernels that run over the M coarse rows, a count known on the device only.
// Sized for the fine count n (M's upper bound), most blocks of a launch would only read
// M and exit, each holding its slot for that load (M is n / 8 on a subdivided set); so
// they take a grid of at most CG_BLOCKS blocks, enough to fill the chip, and walk M in
// grid-sized strides.
constexpr int64_t CG_BLOCKS = 2048;
static unsigned cg_grid(int64_t threads)
{
    const int64_t blocks = (threads + 255) / 256;
    return (unsigned)(blocks < 1 ? 1 : (blocks < CG_BLOCKS ? blocks : CG_BLOCKS));
}

// Pool one coarse voxel's children (at most 8, contiguous in sorted order and in slot
// order): one item per (coarse voxel, channel).  MEAN: the fp32 sum in slot order
// divided by the count, one rounding to the output type; else the maximum (exact).
template <typename T, bool MEAN>
__global__ __launch_bounds__(256) void k_down_reduce(const int32_t *__restrict__ perm,
                                                     const uint32_t *__restrict__ seg,
                                                     const uint32_t *__restrict__ start,
                                                     const uint32_t *__restrict__ total, int64_t n, int c,
                                                     const T *__restrict__ feats, T *__restrict__ out_feats)
{
    const int64_t end = (int64_t)*total * c, stride = (int64_t)gridDim.x * 256;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < end; e += stride) {
        int ci;
        const int64_t m = split_index(e, c, ci);
        const int64_t s0 = start[m];
        float acc = MEAN ? 0.f : -__builtin_huge_valf();
        int cnt = 0;
        for (int q = 0; q < 8; ++q) {
            const int64_t s = s0 + q;
            if (s >= n || (int64_t)seg[s] != m) break;
            const float v = Elem<T>::to_f32(feats[(int64_t)perm[s] * c + ci]);
            acc = MEAN ? acc + v : fmaxf(acc, v);
            ++cnt;
        }
        out_feats[m * c + ci] = Elem<T>::from_f32(MEAN ? acc / (float)cnt : acc);
    }
}

// Operations of the coarse-grouping pipelines below.
enum { COARSE_S2D = 0, COARSE_MAX = 1, COARSE_MEAN = 2 };

// ---------------------------------------------------------------------------
// coarse grouping through an occupancy bitmap (dense coarse key spaces)
// ---------------------------------------------------------------------------
// The coarse cells that hold a fine voxel are the set bits of a bitmap over the
// coarse key space; a cell's rank among them (prefix of the words' popcounts plus
// the bits below it in its word) is its output row, in ascending key order.  Each
// fine voxel then writes its row number into its cell's slot of an 8-entry child
// list, and the output kernels read the children in slot order.  No sort.

constexpr int CG_SLOTS = 2048;  // LDS hash slots per block in the mark (2 x the block's rows)

// Validate, pack the coarse key (all ones for an invalid row) and set its bit; a
// block first ORs its rows' bits into an LDS hash keyed by bitmap word, so that a
// word costs one device-scope atomic per block (children of one cell are usually
// neighbours in the input).
__global__ __launch_bounds__(256) void k_cg_mark(const int4 *__restrict__ coords, int64_t n, int res, int batch,
                                                 int rbc, uint32_t *__restrict__ ckey,
                                                 unsigned long long *__restrict__ bm, DevStatus *st)
{
    __shared__ unsigned long long s_word[CG_SLOTS];
    __shared__ unsigned long long s_bits[CG_SLOTS];
    for (int i = threadIdx.x; i < CG_SLOTS; i += 256) {
        s_word[i] = ~0ull;
        s_bits[i] = 0ull;
    }
    __syncthreads();
    bool bad_any = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int64_t i = (int64_t)blockIdx.x * 1024 + q * 256 + threadIdx.x;
        if (i >= n) continue;
        const int4 c = coords[i];
        const bool bad = (unsigned)c.x >= (unsigned)batch || (unsigned)c.y >= (unsigned)res ||
                         (unsigned)c.z >= (unsigned)res || (unsigned)c.w >= (unsigned)res;
        bad_any |= bad;
        uint32_t key = ~0u;
        if (!bad) {
            key = ((((uint32_t)c.x << rbc | (uint32_t)(c.y >> 1)) << rbc | (uint32_t)(c.z >> 1)) << rbc) |
                  (uint32_t)(c.w >> 1);
            const unsigned long long w = key >> 6;
            uint32_t h = ((uint32_t)w * 0x9E3779B1u) >> (32 - 11);
            for (;;) {  // linear probing; twice as many slots as rows, so it never fills
                const unsigned long long prev = atomicCAS(&s_word[h], ~0ull, w);
                if (prev == ~0ull || prev == w) break;
                h = (h + 1) & (CG_SLOTS - 1);
            }
            atomicOr(&s_bits[h], 1ull << (key & 63));
        }
        ckey[i] = key;
    }
    if (bad_any) atomicOr(&st->flags, FLAG_RANGE);
    __syncthreads();
    for (int i = threadIdx.x; i < CG_SLOTS; i += 256)
        if (s_word[i] != ~0ull) atomicOr(&bm[s_word[i]], s_bits[i]);
}

// Child lists of the M coarse rows to -1.
__global__ __launch_bounds__(256) void k_cg_init(int4 *__restrict__ child, const uint32_t *__restrict__ total)
{
    const int64_t mend = *total, stride = (int64_t)gridDim.x * 256;
    for (int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x; m < mend; m += stride) {
        child[2 * m] = make_int4(-1, -1, -1, -1);
        child[2 * m + 1] = make_int4(-1, -1, -1, -1);
    }
}

// Row of each fine voxel's cell, its slot in the cell's child list (a second voxel
// in one slot is a duplicate), and the cell's coordinates (every child writes the
// same values).
__global__ __launch_bounds__(256) void k_cg_rank(const uint32_t *__restrict__ ckey, const int4 *__restrict__ coords,
                                                 int64_t n, int rbc, const unsigned long long *__restrict__ bm,
                                                 const uint32_t *__restrict__ prefix, int32_t *__restrict__ child,
                                                 int4 *__restrict__ out_coords, DevStatus *st)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const uint32_t key = ckey[i];
    if (key == ~0u) return;
    const uint32_t w = key >> 6;
    const int64_t m = (int64_t)prefix[w] + __popcll(bm[w] & ((1ull << (key & 63)) - 1ull));
    if (m >= n) return;
    const int4 c = coords[i];
    const int slot = (c.y & 1) | ((c.z & 1) << 1) | ((c.w & 1) << 2);
    if (atomicCAS(&child[m * 8 + slot], -1, (int32_t)i) != -1) atomicOr(&st->flags, FLAG_DUPLICATE);
    const uint32_t msk = (1u << rbc) - 1u;
    out_coords[m] = make_int4((int)(key >> (3 * rbc)), (int)((key >> (2 * rbc)) & msk), (int)((key >> rbc) & msk),
                              (int)(key & msk));
}

// Downsample output: one item per (coarse row, group of V channels), V = 16 bytes of
// channels when rows are whole 16-byte vectors, else 1; children in slot order.
template <typename T, int V, bool MEAN>
__device__ __forceinline__ void cg_pool_item(const int32_t *__restrict__ child, int c, const T *__restrict__ feats,
                                             T *__restrict__ out_feats, int64_t m, int gi)
{
    const int c0 = gi * V;
    float acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = MEAN ? 0.f : -__builtin_huge_valf();
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int32_t r = child[m * 8 + q];
        if (r < 0) continue;
        T x[V];
        if constexpr (V * sizeof(T) == 16) *(uint4 *)x = *(const uint4 *)(feats + (int64_t)r * c + c0);
        else x[0] = feats[(int64_t)r * c + c0];
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const float f = Elem<T>::to_f32(x[v]);
            acc[v] = MEAN ? acc[v] + f : fmaxf(acc[v], f);
        }
        ++cnt;
    }
    T y[V];
#pragma unroll
    for (int v = 0; v < V; ++v) y[v] = Elem<T>::from_f32(MEAN ? acc[v] / (float)cnt : acc[v]);
    if constexpr (V * sizeof(T) == 16) *(uint4 *)(out_feats + m * c + c0) = *(const uint4 *)y;
    else out_feats[m * c + c0] = y[0];
}

template <typename T, int V, bool MEAN>
__global__ __launch_bounds__(256) void k_cg_pool(const int32_t *__restrict__ child, const uint32_t *__restrict__ total,
                                                 int c, const T *__restrict__ feats, T *__restrict__ out_feats)
{
    const int groups = c / V;
    const int64_t end = (int64_t)*total * groups, stride = (int64_t)gridDim.x * 256;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < end; e += stride) {
        int gi;
        const int64_t m = split_index(e, groups, gi);
        cg_pool_item<T, V, MEAN>(child, c, feats, out_feats, m, gi);
    }
}

// Space-to-depth output: one item per (coarse row, slot, unit of a row), units U of
// 16 bytes when rows are whole vectors, else elements; empty slots zero.
template <typename U>
__global__ __launch_bounds__(256) void k_cg_s2d(const int32_t *__restrict__ child, const uint32_t *__restrict__ total,
                                                int upr, const U *__restrict__ feats, U *__restrict__ out_feats,
                                                uint8_t *__restrict__ out_mask)
{
    const int64_t end = (int64_t)*total * 8 * upr, stride = (int64_t)gridDim.x * 256;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < end; e += stride) {  // rows x 8 slots x units
        int ui;
        const int64_t ms = split_index(e, upr, ui);
        const int32_t r = child[ms];
        out_feats[e] = r >= 0 ? feats[(int64_t)r * upr + ui] : U{};
        if (ui == 0 && out_mask) out_mask[ms] = r >= 0;
    }
}

template <typename T>
static int coarse_group_bitmap(const int32_t *coords, const void *feats, int64_t n, int c, int res, int batch,
                               int rbc, int nbits, int32_t *out_coords, void *out_feats, uint8_t *out_mask,
                               int64_t *out_m, hipStream_t s, int op)
{
    auto up = [](size_t b) { return (b + 255) & ~size_t(255); };
    const int64_t words = nbits > 6 ? (int64_t(1) << (nbits - 6)) : 1;
    size_t off = 0;
    const size_t o_bm = off; off += up((size_t)(words + 1) * 8);
    const size_t o_pre = off; off += up((size_t)words * 4);
    const size_t o_key = off; off += up((size_t)n * 4);
    const size_t o_child = off; off += up((size_t)n * 32);
    const size_t o_scan = off; off += up(scan_scratch_bytes(words));
    const size_t o_st = off; off += sizeof(DevStatus);
    char *sc = nullptr;
    SC_CHECK(dev_alloc((void **)&sc, off, s));
    unsigned long long *bm = (unsigned long long *)(sc + o_bm);
    uint32_t *pre = (uint32_t *)(sc + o_pre), *ckey = (uint32_t *)(sc + o_key);
    int32_t *child = (int32_t *)(sc + o_child);
    DevStatus *st = (DevStatus *)(sc + o_st);
    uint32_t *total = (uint32_t *)&st->count;
    int status = SUBMCONV_OK;
    do {
        if (hipMemsetAsync(bm, 0, (size_t)(words + 1) * 8, s) != hipSuccess ||
            hipMemsetAsync(st, 0, sizeof(DevStatus), s) != hipSuccess) {
            status = fail(SUBMCONV_E_HIP, "clear failed");
            break;
        }
        hipLaunchKernelGGL(k_cg_mark, dim3((unsigned)((n + 1023) / 1024)), dim3(256), 0, s, (const int4 *)coords, n, res,
                           batch, rbc, ckey, bm, st);
        if ((status = exclusive_scan_u32((const uint32_t *)bm, pre, words, total, sc + o_scan, s, SCAN_POPC64, true)) !=
            SUBMCONV_OK)
            break;
        hipLaunchKernelGGL(k_cg_init, dim3(cg_grid(n)), dim3(256), 0, s, (int4 *)child, total);
        hipLaunchKernelGGL(k_cg_rank, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ckey, (const int4 *)coords, n,
                           rbc, bm, pre, child, (int4 *)out_coords, st);
        constexpr int V = 16 / sizeof(T);  // elements of a 16-byte vector
        const bool vec = (c * sizeof(T)) % 16 == 0 && ((uintptr_t)feats & 15) == 0 && ((uintptr_t)out_feats & 15) == 0;
        if (op == COARSE_S2D) {
            if (vec)
                hipLaunchKernelGGL(k_cg_s2d<uint4>, dim3(cg_grid(n * 8 * (c / V))), dim3(256), 0, s,
                                   child, total, c / V, (const uint4 *)feats, (uint4 *)out_feats, out_mask);
            else
                hipLaunchKernelGGL(k_cg_s2d<T>, dim3(cg_grid(n * 8 * c)), dim3(256), 0, s, child, total,
                                   c, (const T *)feats, (T *)out_feats, out_mask);
        } else {
            const int gv = vec ? V : 1;
            const unsigned grid = cg_grid(n * (c / gv));
            if (vec && op == COARSE_MEAN)
                hipLaunchKernelGGL((k_cg_pool<T, V, true>), dim3(grid), dim3(256), 0, s, child, total, c, (const T *)feats,
                                   (T *)out_feats);
            else if (vec)
                hipLaunchKernelGGL((k_cg_pool<T, V, false>), dim3(grid), dim3(256), 0, s, child, total, c,
                                   (const T *)feats, (T *)out_feats);
            else if (op == COARSE_MEAN)
                hipLaunchKernelGGL((k_cg_pool<T, 1, true>), dim3(grid), dim3(256), 0, s, child, total, c, (const T *)feats,
                                   (T *)out_feats);
            else
                hipLaunchKernelGGL((k_cg_pool<T, 1, false>), dim3(grid), dim3(256), 0, s, child, total, c,
                                   (const T *)feats, (T *)out_feats);
        }
        Mailbox *mb = nullptr;
        uint32_t seq = 0;
        if ((status = mailbox_acquire(&mb, &seq)) != SUBMCONV_OK) break;
        hipLaunchKernelGGL(k_post_count, dim3(1), dim3(1), 0, s, (const uint32_t *)total, (const DevStatus *)st, mb, seq);
        if (hipGetLastError() != hipSuccess) { status = fail(SUBMCONV_E_HIP, "launch in a coarse grouping failed"); break; }
        DevStatus h;
        if ((status = mailbox_wait(mb, seq, &h, s)) != SUBMCONV_OK) break;
        if (h.flags & FLAG_RANGE) status = fail(SUBMCONV_E_COORD_RANGE, "a coordinate is outside [0,res) or its batch index outside [0,batch)");
        else if (h.flags & FLAG_DUPLICATE) status = fail(SUBMCONV_E_DUPLICATE, "the coordinate set holds a duplicate row");
        else *out_m = (int64_t)h.count;
    } while (0);
    dev_free(sc, s);
    return status;
}

template <typename K, typename T>
static int s2d_impl(const int32_t *coords, const void *feats, int64_t n, int c, int res, int batch,
                    int32_t *out_coords, void *out_feats, uint8_t *out_mask, int64_t *out_m,
                    hipStream_t s, int op = COARSE_S2D)
{
    const int rbc = bits_for((res + 1) / 2);
    const int nbits = 3 * rbc + bits_for(batch) + 3;
    // scratch: keys a/b, rows a/b, head, seg, total, sort scratch, scan scratch, status
    auto up = [](size_t b) { return (b + 255) & ~size_t(255); };
    const size_t kb = up((size_t)n * sizeof(K)), vb = up((size_t)n * 4);
    size_t off = 0;
    const size_t o_ka = off; off += kb;
    const size_t o_kb = off; off += kb;
    const size_t o_va = off; off += vb;
    const size_t o_vb = off; off += vb;
    const size_t o_head = off; off += vb;
    const size_t o_seg = off; off += vb;
    const size_t o_start = off; off += op == COARSE_S2D ? 0 : vb;
    const size_t o_tot = off; off += 256;
    const size_t o_sort = off; off += up(sort_scratch_bytes(n));
    const size_t o_scan = off; off += up(scan_scratch_bytes(n));
    const size_t o_st = off; off += sizeof(DevStatus);
    char *sc = nullptr;
    SC_CHECK(dev_alloc((void **)&sc, off, s));
    K *ka = (K *)(sc + o_ka), *kb_ = (K *)(sc + o_kb);
    int32_t *va = (int32_t *)(sc + o_va), *vb_ = (int32_t *)(sc + o_vb);
    uint32_t *head = (uint32_t *)(sc + o_head), *seg = (uint32_t *)(sc + o_seg);
    uint32_t *tot = (uint32_t *)(sc + o_tot);
    DevStatus *st = (DevStatus *)(sc + o_st);
    int status = SUBMCONV_OK;
    do {
        if (hipMemsetAsync(st, 0, sizeof(DevStatus), s) != hipSuccess) { status = fail(SUBMCONV_E_HIP, "status clear failed"); break; }
        const unsigned grid = (unsigned)((n + 255) / 256);
        const bool in_b = radix_sort_passes(n, nbits) & 1;
        hipLaunchKernelGGL(k_s2d_pack<K>, dim3(grid), dim3(256), 0, s, (const int4 *)coords, n, res,
                           batch, rbc, in_b ? kb_ : ka, in_b ? vb_ : va, st);
        if ((status = radix_sort_pairs<K>(ka, va, kb_, vb_, n, nbits, sc + o_sort, s, in_b)) != SUBMCONV_OK) break;
        hipLaunchKernelGGL(k_s2d_heads<K>, dim3(grid), dim3(256), 0, s, ka, n, head, st);
        if ((status = exclusive_scan_u32(head, seg, n, tot, sc + o_scan, s)) != SUBMCONV_OK) break;
        hipLaunchKernelGGL(k_excl_to_seg, dim3(grid), dim3(256), 0, s, head, seg, n);
        const int64_t total = n * c;
        if (op == COARSE_S2D) {
            hipLaunchKernelGGL((k_s2d_rows<K, T>), dim3(grid), dim3(256), 0, s, ka, head, seg, n, rbc, c,
                               (int4 *)out_coords, (T *)out_feats, out_mask);
            hipLaunchKernelGGL((k_s2d_scatter<K, T>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                               s, ka, va, seg, n, c, (const T *)feats, (T *)out_feats, out_mask);
        } else {
            uint32_t *start = (uint32_t *)(sc + o_start);
            hipLaunchKernelGGL(k_down_rows<K>, dim3(grid), dim3(256), 0, s, ka, head, seg, n, rbc,
                               (int4 *)out_coords, start);
            if (op == COARSE_MEAN)
                hipLaunchKernelGGL((k_down_reduce<T, true>), dim3(cg_grid(total)), dim3(256), 0,
                                   s, va, seg, start, tot, n, c, (const T *)feats, (T *)out_feats);
            else
                hipLaunchKernelGGL((k_down_reduce<T, false>), dim3(cg_grid(total)), dim3(256), 0,
                                   s, va, seg, start, tot, n, c, (const T *)feats, (T *)out_feats);
        }
        Mailbox *mb = nullptr;
        uint32_t seq = 0;
        if ((status = mailbox_acquire(&mb, &seq)) != SUBMCONV_OK) break;
        hipLaunchKernelGGL(k_post_count, dim3(1), dim3(1), 0, s, (const uint32_t *)tot, (const DevStatus *)st, mb, seq);
        if (hipGetLastError() != hipSuccess) { status = fail(SUBMCONV_E_HIP, "launch in %s failed", op == COARSE_S2D ? "space_to_depth" : "downsample"); break; }
        DevStatus h;
        if ((status = mailbox_wait(mb, seq, &h, s)) != SUBMCONV_OK) break;
        if (h.flags & FLAG_RANGE) status = fail(SUBMCONV_E_COORD_RANGE, "a coordinate is outside [0,res) or its batch index outside [0,batch)");
        else if (h.flags & FLAG_DUPLICATE) status = fail(SUBMCONV_E_DUPLICATE, "the coordinate set holds a duplicate row");
        else *out_m = (int64_t)h.count;
    } while (0);
    dev_free(sc, s);
    return status;
}

static int coarse_group(const int32_t *coords, const void *feats, int64_t n, int c, int dtype, int res, int batch,
                        int32_t *out_coords, void *out_feats, uint8_t *out_mask, int64_t *out_m, hipStream_t s,
                        int op)
{
    if (n == 0) { *out_m = 0; return SUBMCONV_OK; }
    const int rbc = bits_for((res + 1) / 2);
    const int nbits = 3 * rbc + bits_for(batch) + 3;
    if (nbits > 64) return fail(SUBMCONV_E_UNSUPPORTED, "grid and batch need %d key bits (max 64)", nbits);
    const bool k32 = nbits <= 32;
    // dense coarse key space (the bitmap within a small multiple of the per-voxel data): no sort
    const int cbits = nbits - 3;
    if (cbits <= 31 && (int64_t(1) << cbits) / 8 <= 64 * n + (int64_t(4) << 20)) {
        if (dtype == SUBMCONV_F32)
            return coarse_group_bitmap<float>(coords, feats, n, c, res, batch, rbc, cbits, out_coords, out_feats,
                                              out_mask, out_m, s, op);
        return coarse_group_bitmap<uint16_t>(coords, feats, n, c, res, batch, rbc, cbits, out_coords, out_feats,
                                             out_mask, out_m, s, op);
    }
    if (dtype == SUBMCONV_F32)
        return k32 ? s2d_impl<uint32_t, float>(coords, feats, n, c, res, batch, out_coords, out_feats, out_mask, out_m, s, op)
                   : s2d_impl<uint64_t, float>(coords, feats, n, c, res, batch, out_coords, out_feats, out_mask, out_m, s, op);
    return k32 ? s2d_impl<uint32_t, uint16_t>(coords, feats, n, c, res, batch, out_coords, out_feats, out_mask, out_m, s, op)
               : s2d_impl<uint64_t, uint16_t>(coords, feats, n, c, res, batch, out_coords, out_feats, out_mask, out_m, s, op);
}

int space_to_depth(const int32_t *coords, const void *feats, int64_t n, int c, int dtype, int res,
                   int batch, int32_t *out_coords, void *out_feats, uint8_t *out_mask,
                   int64_t *out_m, hipStream_t s)
{
    return coarse_group(coords, feats, n, c, dtype, res, batch, out_coords, out_feats, out_mask, out_m, s, COARSE_S2D);
}

int downsample(const int32_t *coords, const void *feats, int64_t n, int c, int dtype, int res, int batch,
               int mean, int32_t *out_coords, void *out_feats, int64_t *out_m, hipStream_t s)
{
    return coarse_group(coords, feats, n, c, dtype, res, batch, out_coords, out_feats, nullptr, out_m, s,
                        mean ? COARSE_MEAN : COARSE_MAX);
}

// ---------------------------------------------------------------------------
// depth_to_space
// ---------------------------------------------------------------------------

// Count of emitted children per coarse voxel.
__global__ __launch_bounds__(256) void k_d2s_count(const uint8_t *__restrict__ mask, int64_t m,
                                                   uint32_t *__restrict__ cnt)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= m) return;
    uint32_t c = 0;
    for (int q = 0; q < 8; ++q) c += mask[i * 8 + q] != 0;
    cnt[i] = c;
}

// Mask bits of a voxel's 8 slots (bit q set when mask byte q is nonzero).  MASK8: the
// mask row is 8-byte aligned and read as one word.
template <bool MASK8>
__device__ __forceinline__ uint32_t slot_bits(const uint8_t *__restrict__ mask, int64_t cell)
{
    uint32_t bits = 0;
    if (MASK8) {
        const unsigned long long w = *(const unsigned long long *)(mask + cell * 8);
#pragma unroll
        for (int q = 0; q < 8; ++q) bits |= ((w >> (8 * q)) & 0xFFull) ? 1u << q : 0u;
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) bits |= mask[cell * 8 + q] ? 1u << q : 0u;
    }
    return bits;
}

// Children of the two expansions.  V = uint4 when rows are whole 16-byte vectors, else
// the element type.  mask == nullptr: every slot, child 8 cell + slot; else the masked
// slots, in slot order, from base[cell].
//
// Masked upsample: the child copies the parent's whole row.  One thread per (voxel,
// vector of the row), over the 8 slots in order, so the parent row is read once.
template <typename V, bool MASK8>
__global__ __launch_bounds__(256) void k_expand(const int4 *__restrict__ cc, const V *__restrict__ cf,
                                                const uint8_t *__restrict__ mask, const uint32_t *__restrict__ base,
                                                int64_t m, int vpr, int4 *__restrict__ out_coords,
                                                V *__restrict__ out_feats)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over m x vpr
    if (e >= m * vpr) return;
    int vi;
    const int64_t cell = split_index(e, vpr, vi);
    uint32_t bits = 0xFFu;
    int64_t dst = cell * 8;
    if (mask) {
        bits = slot_bits<MASK8>(mask, cell);
        dst = base[cell];
    }
    const V v = cf[cell * vpr + vi];
    int4 p = make_int4(0, 0, 0, 0);
    if (vi == 0) p = cc[cell];
#pragma unroll
    for (int slot = 0; slot < 8; ++slot) {
        if (!((bits >> slot) & 1u)) continue;
        if (dst >= 8 * m) break;
        out_feats[dst * vpr + vi] = v;
        if (vi == 0)
            out_coords[dst] = make_int4(p.x, 2 * p.y + (slot & 1), 2 * p.z + ((slot >> 1) & 1), 2 * p.w + (slot >> 2));
        ++dst;
    }
}

// depth_to_space: child `slot` takes that slot's channels of the voxel's 8-times-wider
// row.  One thread per (voxel, slot, vector of a child row): thread e copies input
// element e, so a voxel's whole row is read as one contiguous run, and its present
// children, which take consecutive output rows, are written as one.
template <typename V, bool MASK8>
__global__ __launch_bounds__(256) void k_d2s(const int4 *__restrict__ cc, const V *__restrict__ cf,
                                             const uint8_t *__restrict__ mask, const uint32_t *__restrict__ base,
                                             int64_t m, int vpr, int4 *__restrict__ out_coords,
                                             V *__restrict__ out_feats)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over m x 8 x vpr
    if (e >= m * 8 * vpr) return;
    int r, vi;
    const int64_t cell = split_index(e, 8 * vpr, r);
    const int slot = (int)split_index(r, vpr, vi);
    int64_t dst = cell * 8 + slot;
    if (mask) {
        const uint32_t bits = slot_bits<MASK8>(mask, cell);
        if (!((bits >> slot) & 1u)) return;
        dst = base[cell] + __popc(bits & ((1u << slot) - 1u));
        if (dst >= 8 * m) return;
    }
    out_feats[dst * vpr + vi] = cf[e];
    if (vi == 0) {
        const int4 p = cc[cell];
        out_coords[dst] = make_int4(p.x, 2 * p.y + (slot & 1), 2 * p.z + ((slot >> 1) & 1), 2 * p.w + (slot >> 2));
    }
}

template <typename V, bool REPL>
static void launch_expand_v(const int32_t *cc, const V *cf, const uint8_t *mask, const uint32_t *base, int64_t m,
                            int vpr, int32_t *out_coords, V *out_feats, hipStream_t s)
{
    if constexpr (!REPL) {
        const unsigned g8 = (unsigned)((m * 8 * vpr + 255) / 256);
        if (mask && ((uintptr_t)mask & 7) == 0)
            hipLaunchKernelGGL((k_d2s<V, true>), dim3(g8), dim3(256), 0, s, (const int4 *)cc, cf, mask, base, m, vpr,
                               (int4 *)out_coords, out_feats);
        else
            hipLaunchKernelGGL((k_d2s<V, false>), dim3(g8), dim3(256), 0, s, (const int4 *)cc, cf, mask, base, m, vpr,
                               (int4 *)out_coords, out_feats);
    } else {
        const unsigned grid = (unsigned)((m * vpr + 255) / 256);
        if (mask && ((uintptr_t)mask & 7) == 0)
            hipLaunchKernelGGL((k_expand<V, true>), dim3(grid), dim3(256), 0, s, (const int4 *)cc, cf, mask, base, m,
                               vpr, (int4 *)out_coords, out_feats);
        else
            hipLaunchKernelGGL((k_expand<V, false>), dim3(grid), dim3(256), 0, s, (const int4 *)cc, cf, mask, base,
                               m, vpr, (int4 *)out_coords, out_feats);
    }
}

template <bool REPL>
static int launch_expand(const int32_t *cc, const void *cf, const uint8_t *mask, const uint32_t *base, int64_t m,
                          int c, int dtype, int32_t *out_coords, void *out_feats, hipStream_t s)
{
    const int es = dtype == SUBMCONV_F32 ? 4 : 2;
    const int64_t row = (int64_t)c * es;  // bytes of a child row
    const bool vec = row % 16 == 0 && ((uintptr_t)cf & 15) == 0 && ((uintptr_t)out_feats & 15) == 0;
    if (vec)
        launch_expand_v<uint4, REPL>(cc, (const uint4 *)cf, mask, base, m, (int)(row / 16), out_coords,
                                     (uint4 *)out_feats, s);
    else if (dtype == SUBMCONV_F32)
        launch_expand_v<float, REPL>(cc, (const float *)cf, mask, base, m, c, out_coords, (float *)out_feats, s);
    else
        launch_expand_v<uint16_t, REPL>(cc, (const uint16_t *)cf, mask, base, m, c, out_coords, (uint16_t *)out_feats,
                                        s);
    SC_LAUNCHED("expand");
    return SUBMCONV_OK;
}

// Scratch of a masked expansion of m voxels: per-voxel child counts, their exclusive
// scan, the total, the scan's tile sums and a status block.
struct ExpandScratch {
    size_t cnt, base, tot, scan, st, bytes;
    explicit ExpandScratch(int64_t m)
    {
        auto up = [](size_t b) { return (b + 255) & ~size_t(255); };
        cnt = 0;
        base = up((size_t)m * 4);
        tot = base + up((size_t)m * 4);
        scan = tot + 256;
        st = scan + up(scan_scratch_bytes(m));
        bytes = st + sizeof(DevStatus);
    }
};

// Count the flagged slots per voxel, scan the counts and write the children, with the
// scratch at `sc` (ExpandScratch(m).bytes).  Every scratch word that is read is written
// first in the same call, so nothing needs clearing.  The child count ends up in the
// scratch's total word.
template <bool REPL>
static int expand_masked_enqueue(const int32_t *cc, const void *cf, const uint8_t *mask, int64_t m, int c, int dtype,
                                 int32_t *out_coords, void *out_feats, char *sc, hipStream_t s)
{
    const ExpandScratch L(m);
    uint32_t *cnt = (uint32_t *)(sc + L.cnt), *base = (uint32_t *)(sc + L.base), *tot = (uint32_t *)(sc + L.tot);
    hipLaunchKernelGGL(k_d2s_count, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, s, mask, m, cnt);
    SC_CHECK(exclusive_scan_u32(cnt, base, m, tot, sc + L.scan, s));
    return launch_expand<REPL>(cc, cf, mask, base, m, c, dtype, out_coords, out_feats, s);
}

template <bool REPL>
static int expand(const int32_t *cc, const void *cf, const uint8_t *mask, int64_t m, int c, int dtype,
                  int32_t *out_coords, void *out_feats, int64_t *out_n, hipStream_t s)
{
    if (m == 0) { *out_n = 0; return SUBMCONV_OK; }
    if (!mask) {
        const int status = launch_expand<REPL>(cc, cf, nullptr, nullptr, m, c, dtype, out_coords, out_feats, s);
        if (status == SUBMCONV_OK) *out_n = 8 * m;
        return status;
    }
    const ExpandScratch L(m);
    char *sc = nullptr;
    SC_CHECK(dev_alloc((void **)&sc, L.bytes, s));
    int status = SUBMCONV_OK;
    do {
        if ((status = expand_masked_enqueue<REPL>(cc, cf, mask, m, c, dtype, out_coords, out_feats, sc, s)) !=
            SUBMCONV_OK) break;
        Mailbox *mb = nullptr;
        uint32_t seq = 0;
        if ((status = mailbox_acquire(&mb, &seq)) != SUBMCONV_OK) break;
        hipLaunchKernelGGL(k_post_count, dim3(1), dim3(1), 0, s, (const uint32_t *)(sc + L.tot), (const DevStatus *)nullptr,
                           mb, seq);
        if (hipGetLastError() != hipSuccess) { status = fail(SUBMCONV_E_HIP, "launch in a masked expansion failed"); break; }
        DevStatus h;
        if ((status = mailbox_wait(mb, seq, &h, s)) != SUBMCONV_OK) break;
        *out_n = (int64_t)h.count;
    } while (0);
    dev_free(sc, s);
    return status;
}

// ---------------------------------------------------------------------------
// the masked upsample without allocation
// ---------------------------------------------------------------------------

// The scratch of submconv_upsample_masked_noalloc: one fixed array per device, held
// until the process ends.  Host code must not pass `scratch` itself to a kernel (on
// the host it is a stand-in for the symbol, not a device address): its device
// address is looked up once per device with hipGetSymbolAddress and kept in
// g_scratch_dev.
constexpr size_t NOALLOC_SCRATCH_BYTES = SUBMCONV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];
static std::mutex g_scratch_mu;
static char *g_scratch_dev[64];

static int noalloc_scratch(char **p)
{
    int dev = 0;
    SC_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= 64) return fail(SUBMCONV_E_UNSUPPORTED, "device %d", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *q = nullptr;
        const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !q)
            return fail(SUBMCONV_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_dev[dev] = (char *)q;
    }
    *p = g_scratch_dev[dev];
    return SUBMCONV_OK;
}

size_t noalloc_expand_bytes(int64_t m) { return ExpandScratch(m).bytes; }

int upsample_masked_noalloc(const int32_t *coords, const void *feats, const uint8_t *mask, int64_t n, int c,
                            int dtype, int32_t *out_coords, void *out_feats, int64_t *out_n, hipStream_t s)
{
    if (n == 0) { *out_n = 0; return SUBMCONV_OK; }
    if (ExpandScratch(n).bytes > NOALLOC_SCRATCH_BYTES)
        return fail(SUBMCONV_E_UNSUPPORTED, "n = %lld needs more than the %zu scratch bytes", (long long)n,
                    NOALLOC_SCRATCH_BYTES);
    char *sc = nullptr;
    SC_CHECK(noalloc_scratch(&sc));
    SC_CHECK(expand_masked_enqueue<true>(coords, feats, mask, n, c, dtype, out_coords, out_feats, sc, s));
    uint32_t total = 0;  // pageable host word: no pinned staging block is allocated
    SC_HIP(hipMemcpyAsync(&total, sc + ExpandScratch(n).tot, sizeof(total), hipMemcpyDeviceToHost, s));
    SC_HIP(hipStreamSynchronize(s));
    *out_n = (int64_t)total;
    return SUBMCONV_OK;
}

int depth_to_space(const int32_t *cc, const void *cf, const uint8_t *mask, int64_t m, int c,
                   int dtype, int32_t *out_coords, void *out_feats, int64_t *out_n, hipStream_t s)
{
    return expand<false>(cc, cf, mask, m, c, dtype, out_coords, out_feats, out_n, s);
}

int upsample_masked(const int32_t *coords, const void *feats, const uint8_t *mask, int64_t n, int c, int dtype,
                    int32_t *out_coords, void *out_feats, int64_t *out_n, hipStream_t s)
{
    return expand<true>(coords, feats, mask, n, c, dtype, out_coords, out_feats, out_n, s);
}

}  // namespace sc
