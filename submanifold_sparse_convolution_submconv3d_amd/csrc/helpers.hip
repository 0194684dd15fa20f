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

// Copy each parent row to its 8 children, in 4-byte words (rows are whole words).
__global__ __launch_bounds__(256) void k_subdivide_feats(const uint32_t *__restrict__ in,
                                                         int64_t n, int words,
                                                         uint32_t *__restrict__ out)
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
        if (row_bytes % 4 == 0) {
            const int words = (int)(row_bytes / 4);
            const int64_t total = kids * words;
            hipLaunchKernelGGL(k_subdivide_feats, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
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

template <typename K, typename T>
static int s2d_impl(const int32_t *coords, const void *feats, int64_t n, int c, int res, int batch,
                    int32_t *out_coords, void *out_feats, uint8_t *out_mask, int64_t *out_m,
                    hipStream_t s)
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
        hipLaunchKernelGGL((k_s2d_rows<K, T>), dim3(grid), dim3(256), 0, s, ka, head, seg, n, rbc, c,
                           (int4 *)out_coords, (T *)out_feats, out_mask);
        const int64_t total = n * c;
        hipLaunchKernelGGL((k_s2d_scatter<K, T>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                           s, ka, va, seg, n, c, (const T *)feats, (T *)out_feats, out_mask);
        hipLaunchKernelGGL(k_store_count, dim3(1), dim3(1), 0, s, tot, st);
        if (hipGetLastError() != hipSuccess) { status = fail(SUBMCONV_E_HIP, "launch in space_to_depth failed"); break; }
        DevStatus h;
        if ((status = read_status(st, &h, s)) != SUBMCONV_OK) break;
        if (h.flags & FLAG_RANGE) status = fail(SUBMCONV_E_COORD_RANGE, "a coordinate is outside [0,res) or its batch index outside [0,batch)");
        else if (h.flags & FLAG_DUPLICATE) status = fail(SUBMCONV_E_DUPLICATE, "the coordinate set holds a duplicate row");
        else *out_m = (int64_t)h.count;
    } while (0);
    dev_free(sc, s);
    return status;
}

int space_to_depth(const int32_t *coords, const void *feats, int64_t n, int c, int dtype, int res,
                   int batch, int32_t *out_coords, void *out_feats, uint8_t *out_mask,
                   int64_t *out_m, hipStream_t s)
{
    if (n == 0) { *out_m = 0; return SUBMCONV_OK; }
    const int rbc = bits_for((res + 1) / 2);
    const int nbits = 3 * rbc + bits_for(batch) + 3;
    if (nbits > 64) return fail(SUBMCONV_E_UNSUPPORTED, "grid and batch need %d key bits (max 64)", nbits);
    const bool k32 = nbits <= 32;
    if (dtype == SUBMCONV_F32)
        return k32 ? s2d_impl<uint32_t, float>(coords, feats, n, c, res, batch, out_coords, out_feats, out_mask, out_m, s)
                   : s2d_impl<uint64_t, float>(coords, feats, n, c, res, batch, out_coords, out_feats, out_mask, out_m, s);
    return k32 ? s2d_impl<uint32_t, uint16_t>(coords, feats, n, c, res, batch, out_coords, out_feats, out_mask, out_m, s)
               : s2d_impl<uint64_t, uint16_t>(coords, feats, n, c, res, batch, out_coords, out_feats, out_mask, out_m, s);
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

// One thread per (coarse voxel, slot, channel); base == nullptr means all slots.
template <typename T>
__global__ __launch_bounds__(256) void k_d2s_emit(const int4 *__restrict__ cc,
                                                  const T *__restrict__ cf,
                                                  const uint8_t *__restrict__ mask,
                                                  const uint32_t *__restrict__ base, int64_t m,
                                                  int c, int4 *__restrict__ out_coords,
                                                  T *__restrict__ out_feats)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over m x 8 x c
    if (e >= m * 8 * c) return;
    const int64_t cell = e / (8 * c);
    const int rest = (int)(e - cell * 8 * c);
    const int slot = rest / c, ci = rest - slot * c;
    int64_t dst;
    if (mask) {
        if (!mask[cell * 8 + slot]) return;
        int before = 0;
        for (int q = 0; q < slot; ++q) before += mask[cell * 8 + q] != 0;
        dst = (int64_t)base[cell] + before;
        if (dst >= 8 * m) return;
    } else {
        dst = cell * 8 + slot;
    }
    out_feats[dst * c + ci] = cf[e];
    if (ci == 0) {
        const int4 p = cc[cell];
        out_coords[dst] = make_int4(p.x, 2 * p.y + (slot & 1), 2 * p.z + ((slot >> 1) & 1),
                                    2 * p.w + (slot >> 2));
    }
}

int depth_to_space(const int32_t *cc, const void *cf, const uint8_t *mask, int64_t m, int c,
                   int dtype, int32_t *out_coords, void *out_feats, int64_t *out_n, hipStream_t s)
{
    if (m == 0) { *out_n = 0; return SUBMCONV_OK; }
    const int64_t total = m * 8 * c;
    const unsigned grid = (unsigned)((total + 255) / 256);
    if (!mask) {
        if (dtype == SUBMCONV_F32)
            hipLaunchKernelGGL(k_d2s_emit<float>, dim3(grid), dim3(256), 0, s, (const int4 *)cc,
                               (const float *)cf, nullptr, nullptr, m, c, (int4 *)out_coords, (float *)out_feats);
        else
            hipLaunchKernelGGL(k_d2s_emit<uint16_t>, dim3(grid), dim3(256), 0, s, (const int4 *)cc,
                               (const uint16_t *)cf, nullptr, nullptr, m, c, (int4 *)out_coords, (uint16_t *)out_feats);
        SC_LAUNCHED("d2s_emit");
        *out_n = 8 * m;
        return SUBMCONV_OK;
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
        if (dtype == SUBMCONV_F32)
            hipLaunchKernelGGL(k_d2s_emit<float>, dim3(grid), dim3(256), 0, s, (const int4 *)cc,
                               (const float *)cf, mask, base, m, c, (int4 *)out_coords, (float *)out_feats);
        else
            hipLaunchKernelGGL(k_d2s_emit<uint16_t>, dim3(grid), dim3(256), 0, s, (const int4 *)cc,
                               (const uint16_t *)cf, mask, base, m, c, (int4 *)out_coords, (uint16_t *)out_feats);
        hipLaunchKernelGGL(k_store_count, dim3(1), dim3(1), 0, s, tot, st);
        if (hipGetLastError() != hipSuccess) { status = fail(SUBMCONV_E_HIP, "launch in depth_to_space failed"); break; }
        DevStatus h;
        if ((status = read_status(st, &h, s)) != SUBMCONV_OK) break;
        *out_n = (int64_t)h.count;
    } while (0);
    dev_free(sc, s);
    return status;
}

}  // namespace sc
