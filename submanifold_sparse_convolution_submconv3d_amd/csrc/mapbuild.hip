// Neighbour-map ("rulebook") builder for the submanifold 3x3x3 convolution.
//
// The pages resolve neighbours through a sorted key array with 27 lookups per
// voxel, cached per coordinate set (lato.2_mrp_mlx working notes, commit
// summary).  On gfx950 the build is:
//   pack     - validate (b, z, y, x) and pack it into an integer key
//              ((b << 3rb) | (z << 2rb) | (y << rb) | x), row index as payload;
//   sort     - device LSD radix sort over the significant key bits only;
//   resolve  - per sorted voxel: duplicate check against the next key; the
//              x-neighbours of the centre row are the adjacent sorted entries;
//              each of the other 8 (dz, dy) rows needs one binary search for
//              its x-1 start, then at most two steps forward; results are
//              staged in LDS and written as whole rows of the [N,27] table.
// Coordinates are range-checked before packing and every neighbour coordinate
// is bounds-checked before its key is formed, so a key never wraps into the
// next row, plane or batch entry.
#include "common.h"

namespace sc {

template <typename K>
__global__ __launch_bounds__(256) void k_pack(const int4 *__restrict__ coords, int64_t n, int res,
                                              int batch, int rb, K *__restrict__ keys,
                                              int32_t *__restrict__ rows, DevStatus *st)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int4 c = coords[i];  // (b, z, y, x)
    const bool bad = (unsigned)c.x >= (unsigned)batch || (unsigned)c.y >= (unsigned)res ||
                     (unsigned)c.z >= (unsigned)res || (unsigned)c.w >= (unsigned)res;
    K key = K(0);
    if (!bad) key = ((((K)c.x << rb | (K)c.y) << rb | (K)c.z) << rb) | (K)c.w;
    keys[i] = key;
    rows[i] = (int32_t)i;
    if (bad) atomicOr(&st->flags, FLAG_RANGE);
}

template <typename K>
__device__ __forceinline__ int64_t lower_bound_key(const K *__restrict__ a, int64_t n, K t)
{
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (a[mid] < t) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

template <typename K>
__global__ __launch_bounds__(256) void k_resolve(const K *__restrict__ sk,
                                                 const int32_t *__restrict__ perm, int64_t n,
                                                 int res, int rb, int32_t *__restrict__ nbr,
                                                 DevStatus *st)
{
    __shared__ int32_t s_rows[256 * 27];
    __shared__ int32_t s_dst[256];
    __shared__ uint32_t s_red[4];

    const int64_t s0 = (int64_t)blockIdx.x * 256;
    const int64_t s = s0 + threadIdx.x;
    const int count = (int)((n - s0) < 256 ? (n - s0) : 256);
    uint32_t present = 0;
    bool dup = false;
    if (s < n) {
        const K key = sk[s];
        const K m = (K(1) << rb) - 1;
        const int x = (int)(key & m), y = (int)((key >> rb) & m), z = (int)((key >> (2 * rb)) & m);
        const K bpart = (key >> (3 * rb)) << (3 * rb);
        dup = (s + 1 < n) && sk[s + 1] == key;
        int32_t *row = s_rows + threadIdx.x * 27;
        for (int dz = -1; dz <= 1; ++dz) {
            for (int dy = -1; dy <= 1; ++dy) {
                const int kb = 9 * (dz + 1) + 3 * (dy + 1);
                const int nz = z + dz, ny = y + dy;
                if (nz < 0 || nz >= res || ny < 0 || ny >= res) {
                    row[kb] = row[kb + 1] = row[kb + 2] = -1;
                    continue;
                }
                if (dz == 0 && dy == 0) {  // centre row: adjacent sorted entries
                    row[kb] = (x > 0 && s > 0 && sk[s - 1] == key - 1) ? perm[s - 1] : -1;
                    row[kb + 1] = perm[s];
                    row[kb + 2] = (x + 1 < res && s + 1 < n && sk[s + 1] == key + 1) ? perm[s + 1] : -1;
                    continue;
                }
                const K rowkey = bpart | ((K)nz << (2 * rb)) | ((K)ny << rb);
                int64_t p = lower_bound_key(sk, n, rowkey | (K)(x > 0 ? x - 1 : 0));
                for (int dx = -1; dx <= 1; ++dx) {
                    const int nx = x + dx;
                    int32_t r = -1;
                    if (nx >= 0 && nx < res) {
                        const K t = rowkey | (K)nx;
                        while (p < n && sk[p] < t) ++p;
                        if (p < n && sk[p] == t) r = perm[p];
                    }
                    row[kb + dx + 1] = r;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < 27; ++k) present += row[k] >= 0;
        s_dst[threadIdx.x] = perm[s];
    }
    if (dup) atomicOr(&st->flags, FLAG_DUPLICATE);
    uint32_t total;
    block_incl_scan256(present, s_red, &total);  // also a barrier for s_rows / s_dst
    if (threadIdx.x == 0 && total) atomicAdd(&st->taps, (unsigned long long)total);
    // whole rows of the table: consecutive threads write consecutive entries
    for (int e = threadIdx.x; e < count * 27; e += 256) {
        const int r = e / 27, k = e - r * 27;
        const uint32_t dst = (uint32_t)s_dst[r];
        if (dst < (uint64_t)n) nbr[(int64_t)dst * 27 + k] = s_rows[e];
    }
}

template <typename K>
static int build_map_impl(const int32_t *coords, submconv_rulebook *rb, hipStream_t stream)
{
    const int64_t n = rb->n;
    const size_t key_bytes = (size_t)n * sizeof(K);
    // scratch: alternate keys / rows for the sort, sort histograms, status
    const size_t off_vals = (key_bytes + 255) & ~size_t(255);
    const size_t off_sort = off_vals + (((size_t)n * 4 + 255) & ~size_t(255));
    const size_t off_stat = off_sort + ((sort_scratch_bytes(n) + 255) & ~size_t(255));
    const size_t scratch_bytes = off_stat + sizeof(DevStatus);
    char *scratch = nullptr;
    SC_CHECK(dev_alloc((void **)&scratch, scratch_bytes, stream));
    K *keys_b = (K *)scratch;
    int32_t *vals_b = (int32_t *)(scratch + off_vals);
    DevStatus *st = (DevStatus *)(scratch + off_stat);
    int status = SUBMCONV_OK;
    do {
        if (hipMemsetAsync(st, 0, sizeof(DevStatus), stream) != hipSuccess) {
            status = fail(SUBMCONV_E_HIP, "status clear failed");
            break;
        }
        const unsigned grid = (unsigned)((n + 255) / 256);
        hipLaunchKernelGGL(k_pack<K>, dim3(grid), dim3(256), 0, stream, (const int4 *)coords, n,
                           rb->res, rb->batch, rb->rb, (K *)rb->keys, rb->perm, st);
        if (hipGetLastError() != hipSuccess) { status = fail(SUBMCONV_E_HIP, "launch of pack failed"); break; }
        status = radix_sort_pairs<K>((K *)rb->keys, rb->perm, keys_b, vals_b, n, rb->nbits,
                                     scratch + off_sort, stream);
        if (status != SUBMCONV_OK) break;
        hipLaunchKernelGGL(k_resolve<K>, dim3(grid), dim3(256), 0, stream, (const K *)rb->keys,
                           rb->perm, n, rb->res, rb->rb, rb->nbr, st);
        if (hipGetLastError() != hipSuccess) { status = fail(SUBMCONV_E_HIP, "launch of resolve failed"); break; }
        DevStatus h;
        status = read_status(st, &h, stream);
        if (status != SUBMCONV_OK) break;
        if (h.flags & FLAG_RANGE) status = fail(SUBMCONV_E_COORD_RANGE, "a coordinate is outside [0,res) or its batch index outside [0,batch)");
        else if (h.flags & FLAG_DUPLICATE) status = fail(SUBMCONV_E_DUPLICATE, "the coordinate set holds a duplicate row");
        rb->taps = (int64_t)h.taps;
    } while (0);
    dev_free(scratch, stream);
    return status;
}

int build_map(const int32_t *coords, submconv_rulebook *rb, hipStream_t stream)
{
    return rb->key_bytes == 4 ? build_map_impl<uint32_t>(coords, rb, stream)
                              : build_map_impl<uint64_t>(coords, rb, stream);
}

}  // namespace sc
