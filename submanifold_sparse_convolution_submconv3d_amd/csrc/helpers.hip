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
#include "common.h"

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

// Copy each parent row to its 8 children in units V (16-byte vectors or 4-byte words;
// rows are whole units).
template <typename V>
__global__ __launch_bounds__(256) void k_subdivide_feats(const V *__restrict__ in, int64_t n, int words,
                                                         V *__restrict__ out)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over 8n rows x words
    if (e >= 8 * n * words) return;
    const int64_t child = e / words;
    const int wi = (int)(e - child * words);
    out[e] = in[(child >> 3) * words + wi];
}

// 2-byte rows that are not whole words (odd bf16 channel counts)
__global__ __launch_bounds__(256) void k_subdivide_feats16(const uint16_t *__restrict__ in,
                                                           int64_t n, int c,
                                                           uint16_t *__restrict__ out)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= 8 * n * c) return;
    const int64_t child = e / c;
    const int ci = (int)(e - child * c);
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
    const int64_t s = e / c;
    const int ci = (int)(e - s * c);
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

__global__ void k_store_count(const uint32_t *__restrict__ total, DevStatus *st)
{
    st->count = *total;
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

// Pool one coarse voxel's children (at most 8, contiguous in sorted order and in slot
// order): one thread per (coarse voxel, channel).  MEAN: the fp32 sum in slot order
// divided by the count, one rounding to the output type; else the maximum (exact).
template <typename T, bool MEAN>
__global__ __launch_bounds__(256) void k_down_reduce(const int32_t *__restrict__ perm,
                                                     const uint32_t *__restrict__ seg,
                                                     const uint32_t *__restrict__ start,
                                                     const uint32_t *__restrict__ total, int64_t n, int c,
                                                     const T *__restrict__ feats, T *__restrict__ out_feats)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over (at most n coarse voxels) x c
    const int64_t m = e / c;
    if (m >= (int64_t)*total) return;
    const int ci = (int)(e - m * c);
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

// Operations of the coarse-grouping pipeline below.
enum { COARSE_S2D = 0, COARSE_MAX = 1, COARSE_MEAN = 2 };

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
                hipLaunchKernelGGL((k_down_reduce<T, true>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                                   s, va, seg, start, tot, n, c, (const T *)feats, (T *)out_feats);
            else
                hipLaunchKernelGGL((k_down_reduce<T, false>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                                   s, va, seg, start, tot, n, c, (const T *)feats, (T *)out_feats);
        }
        hipLaunchKernelGGL(k_store_count, dim3(1), dim3(1), 0, s, tot, st);
        if (hipGetLastError() != hipSuccess) { status = fail(SUBMCONV_E_HIP, "launch in %s failed", op == COARSE_S2D ? "space_to_depth" : "downsample"); break; }
        DevStatus h;
        if ((status = read_status(st, &h, s)) != SUBMCONV_OK) break;
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

// Children of the two expansions: one thread per (voxel, slot, vector of a child row),
// V = uint4 when rows are whole 16-byte vectors, else the element type.  REPL: the
// child copies the parent's whole row (masked upsample); otherwise it takes the
// slot's channels of an 8-times-wider row (depth_to_space).  mask == nullptr: every
// slot, child 8 cell + slot; else the masked slots at base[cell] + (masked slots before).
template <typename V, bool REPL>
__global__ __launch_bounds__(256) void k_expand(const int4 *__restrict__ cc, const V *__restrict__ cf,
                                                const uint8_t *__restrict__ mask, const uint32_t *__restrict__ base,
                                                int64_t m, int vpr, int4 *__restrict__ out_coords,
                                                V *__restrict__ out_feats)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over m x 8 x vpr
    if (e >= m * 8 * vpr) return;
    const int64_t cell = e / (8 * vpr);
    const int rest = (int)(e - cell * 8 * vpr);
    const int slot = rest / vpr, vi = rest - slot * vpr;
    int64_t dst;
    if (mask) {
        const uint8_t *mr = mask + cell * 8;
        if (!mr[slot]) return;
        int before = 0;
        for (int q = 0; q < slot; ++q) before += mr[q] != 0;
        dst = (int64_t)base[cell] + before;
        if (dst >= 8 * m) return;
    } else {
        dst = cell * 8 + slot;
    }
    out_feats[dst * vpr + vi] = REPL ? cf[cell * vpr + vi] : cf[e];
    if (vi == 0) {
        const int4 p = cc[cell];
        out_coords[dst] = make_int4(p.x, 2 * p.y + (slot & 1), 2 * p.z + ((slot >> 1) & 1), 2 * p.w + (slot >> 2));
    }
}

template <bool REPL>
static int launch_expand(const int32_t *cc, const void *cf, const uint8_t *mask, const uint32_t *base, int64_t m,
                          int c, int dtype, int32_t *out_coords, void *out_feats, hipStream_t s)
{
    const int es = dtype == SUBMCONV_F32 ? 4 : 2;
    const int64_t row = (int64_t)c * es;  // bytes of a child row
    const bool vec = row % 16 == 0 && ((uintptr_t)cf & 15) == 0 && ((uintptr_t)out_feats & 15) == 0;
    const int vpr = vec ? (int)(row / 16) : c;
    const unsigned grid = (unsigned)((m * 8 * vpr + 255) / 256);
    if (vec)
        hipLaunchKernelGGL((k_expand<uint4, REPL>), dim3(grid), dim3(256), 0, s, (const int4 *)cc, (const uint4 *)cf,
                           mask, base, m, vpr, (int4 *)out_coords, (uint4 *)out_feats);
    else if (dtype == SUBMCONV_F32)
        hipLaunchKernelGGL((k_expand<float, REPL>), dim3(grid), dim3(256), 0, s, (const int4 *)cc, (const float *)cf,
                           mask, base, m, vpr, (int4 *)out_coords, (float *)out_feats);
    else
        hipLaunchKernelGGL((k_expand<uint16_t, REPL>), dim3(grid), dim3(256), 0, s, (const int4 *)cc,
                           (const uint16_t *)cf, mask, base, m, vpr, (int4 *)out_coords, (uint16_t *)out_feats);
    SC_LAUNCHED("expand");
    return SUBMCONV_OK;
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
    auto up = [](size_t b) { return (b + 255) & ~size_t(255); };
    const size_t o_cnt = 0, o_base = up((size_t)m * 4), o_tot = o_base + up((size_t)m * 4);
    const size_t o_scan = o_tot + 256, o_st = o_scan + up(scan_scratch_bytes(m));
    char *sc = nullptr;
    SC_CHECK(dev_alloc((void **)&sc, o_st + sizeof(DevStatus), s));
    uint32_t *cnt = (uint32_t *)(sc + o_cnt), *base = (uint32_t *)(sc + o_base), *tot = (uint32_t *)(sc + o_tot);
    DevStatus *st = (DevStatus *)(sc + o_st);
    int status = SUBMCONV_OK;
    do {
        if (hipMemsetAsync(st, 0, sizeof(DevStatus), s) != hipSuccess) { status = fail(SUBMCONV_E_HIP, "status clear failed"); break; }
        hipLaunchKernelGGL(k_d2s_count, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, s, mask, m, cnt);
        if ((status = exclusive_scan_u32(cnt, base, m, tot, sc + o_scan, s)) != SUBMCONV_OK) break;
        if ((status = launch_expand<REPL>(cc, cf, mask, base, m, c, dtype, out_coords, out_feats, s)) != SUBMCONV_OK) break;
        hipLaunchKernelGGL(k_store_count, dim3(1), dim3(1), 0, s, tot, st);
        if (hipGetLastError() != hipSuccess) { status = fail(SUBMCONV_E_HIP, "launch in a masked expansion failed"); break; }
        DevStatus h;
        if ((status = read_status(st, &h, s)) != SUBMCONV_OK) break;
        *out_n = (int64_t)h.count;
    } while (0);
    dev_free(sc, s);
    return status;
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
