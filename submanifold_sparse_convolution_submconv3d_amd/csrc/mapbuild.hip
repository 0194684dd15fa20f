// Neighbour-map ("rulebook") builder for the submanifold 3x3x3 convolution.
//
// The pages resolve neighbours through a sorted key array with 27 lookups per
// voxel, cached per coordinate set (lato.2_mrp_mlx working notes, commit
// summary).  Every coordinate is validated and packed into an integer key
// ((b << 3rb) | (z << 2rb) | (y << rb) | x); keys are sorted, and each voxel's
// 27 neighbour keys are looked up in the sorted order.  Two device strategies:
//
// Dense key space (2^nbits bits of occupancy bitmap affordable next to N):
//   mark     - set the key's bit in an occupancy bitmap (atomicOr); a bit that
//              was already set is a duplicate coordinate;
//   scan     - exclusive scan of the bitmap words' popcounts;
//   rank     - a key's sorted position is prefix[word] + popcount of the lower
//              bits of its word: one radix pass whose digit is the whole key
//              (histogram = bitmap, counts are 0/1 because keys are distinct);
//              scatter key and row to their sorted position;
//   resolve  - per voxel, in input row order, each neighbour is a bit test and,
//              when set, the same rank query plus one read of the row at that
//              sorted position.  The block's 256 table rows are contiguous and
//              are written through LDS as one coalesced run.
//
// Sparse key space (huge grid, few voxels):
//   pack + multi-pass LSD radix sort over the significant key bits, then a
//   windowed resolve: per block of 256 consecutive sorted voxels, the x
//   neighbours of the centre row are the adjacent sorted entries; for each of
//   the other 8 (dz, dy) rows every target key of the block lies in
//   [first + off - 1, last + off + 1] (off = that row's key offset), so the block
//   copies that window of the sorted array into LDS and resolves its voxels by
//   binary search there (a window too big for LDS is searched in place).
//
// Small sets (n <= 2048) run in one block and one launch.  Coordinates are
// range-checked before packing and every neighbour coordinate is bounds-checked
// before its key is formed, so a key never wraps into the next row, plane or
// batch entry.
#include "common.h"

namespace sc {

constexpr int WIN_MAX = 2048;      // window keys held in LDS
constexpr int SMALL_N = 2048;      // single-block build up to this many voxels

template <typename K>
__device__ __forceinline__ K pack_key(int b, int z, int y, int x, int rb)
{
    return ((((K)b << rb | (K)z) << rb | (K)y) << rb) | (K)x;
}

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
    keys[i] = bad ? K(0) : pack_key<K>(c.x, c.y, c.z, c.w, rb);
    rows[i] = (int32_t)i;
    if (bad) atomicOr(&st->flags, FLAG_RANGE);
}

// first index in a[0, n) with a[i] >= t
template <typename K>
__device__ __forceinline__ int64_t lower_bound_key(const K *a, int64_t n, K t)
{
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (a[mid] < t) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// a + delta, clamped to [0, max of K]
template <typename K>
__device__ __forceinline__ K add_sat(K a, int64_t delta)
{
    if (delta < 0) {
        const K d = (K)(-delta);
        return a < d ? K(0) : a - d;
    }
    const K d = (K)delta;
    return a > (K)~K(0) - d ? (K)~K(0) : a + d;
}

template <typename K>
__global__ __launch_bounds__(256) void k_resolve_win(const K *__restrict__ sk,
                                                     const int32_t *__restrict__ perm, int64_t n,
                                                     int res, int rb, int32_t *__restrict__ nbr,
                                                     DevStatus *st)
{
    __shared__ K s_win[WIN_MAX];
    __shared__ int32_t s_wrow[WIN_MAX];
    __shared__ int32_t s_rows[256 * 27];
    __shared__ int32_t s_dst[256];
    __shared__ int64_t s_lo[8], s_hi[8];
    __shared__ uint32_t s_red[4];

    const int tid = threadIdx.x;
    const int64_t s0 = (int64_t)blockIdx.x * 256;
    const int count = (int)((n - s0) < 256 ? (n - s0) : 256);
    const int64_t s = s0 + tid;
    const bool valid = tid < count;
    const K m = (K(1) << rb) - 1;
    const K key = valid ? sk[s] : K(0);
    const int x = (int)(key & m), y = (int)((key >> rb) & m), z = (int)((key >> (2 * rb)) & m);
    const K bpart = (key >> (3 * rb)) << (3 * rb);
    int32_t *row = s_rows + tid * 27;

    // window bounds of the 8 off-centre (dz, dy) rows: 16 binary searches, one per thread
    if (tid < 16) {
        int d = tid >> 1;
        d += (d >= 4);  // skip the centre row (dz, dy) = (0, 0), index 4 of 9
        const int dz = d / 3 - 1, dy = d % 3 - 1;
        const int64_t off = (int64_t)dz * ((int64_t)1 << (2 * rb)) + (int64_t)dy * ((int64_t)1 << rb);
        const K first = sk[s0], last = sk[s0 + count - 1];
        int64_t r;
        if ((tid & 1) == 0) r = lower_bound_key(sk, n, add_sat(first, off - 1));
        else {
            const K t = add_sat(last, off + 1);  // first index with a key > t
            r = (t == (K)~K(0)) ? n : lower_bound_key(sk, n, (K)(t + 1));
        }
        if ((tid & 1) == 0) s_lo[tid >> 1] = r;
        else s_hi[tid >> 1] = r;
    }

    // centre row: adjacent sorted entries
    uint32_t present = 0;
    bool dup = false;
    if (valid) {
        dup = (s + 1 < n) && sk[s + 1] == key;
        row[12] = (x > 0 && s > 0 && sk[s - 1] == key - 1) ? perm[s - 1] : -1;
        row[13] = perm[s];
        row[14] = (x + 1 < res && s + 1 < n && sk[s + 1] == key + 1) ? perm[s + 1] : -1;
        s_dst[tid] = perm[s];
    }
    __syncthreads();

    for (int w = 0; w < 8; ++w) {
        const int d = w + (w >= 4);
        const int dz = d / 3 - 1, dy = d % 3 - 1;
        const int kb = 9 * (dz + 1) + 3 * (dy + 1);
        const int64_t lo = s_lo[w], hi = s_hi[w];
        const int64_t wn = hi - lo;
        const bool in_lds = wn <= WIN_MAX;
        if (in_lds) {
            for (int i = tid; i < wn; i += 256) {
                s_win[i] = sk[lo + i];
                s_wrow[i] = perm[lo + i];
            }
        }
        __syncthreads();
        if (valid) {
            const int nz = z + dz, ny = y + dy;
            if (nz < 0 || nz >= res || ny < 0 || ny >= res) {
                row[kb] = row[kb + 1] = row[kb + 2] = -1;
            } else {
                const K rowkey = bpart | ((K)nz << (2 * rb)) | ((K)ny << rb);
                const K t0 = rowkey | (K)(x > 0 ? x - 1 : 0);
                int64_t p = in_lds ? lower_bound_key(s_win, wn, t0) : lower_bound_key(sk + lo, wn, t0);
                for (int dx = -1; dx <= 1; ++dx) {
                    const int nx = x + dx;
                    int32_t r = -1;
                    if (nx >= 0 && nx < res) {
                        const K t = rowkey | (K)nx;
                        if (in_lds) {
                            while (p < wn && s_win[p] < t) ++p;
                            if (p < wn && s_win[p] == t) r = s_wrow[p];
                        } else {
                            while (p < wn && sk[lo + p] < t) ++p;
                            if (p < wn && sk[lo + p] == t) r = perm[lo + p];
                        }
                    }
                    row[kb + dx + 1] = r;
                }
            }
        }
        __syncthreads();
    }
    if (valid) {
#pragma unroll
        for (int k = 0; k < 27; ++k) present += row[k] >= 0;
    }
    if (dup) atomicOr(&st->flags, FLAG_DUPLICATE);
    uint32_t total;
    block_incl_scan256(present, s_red, &total);  // also a barrier for s_rows / s_dst
    if (tid == 0 && total) atomicAdd(&st->taps, (unsigned long long)total);
    for (int e = tid; e < count * 27; e += 256) {
        const int r = e / 27, k = e - r * 27;
        const uint32_t dst = (uint32_t)s_dst[r];
        if (dst < (uint64_t)n) nbr[(int64_t)dst * 27 + k] = s_rows[e];
    }
}

// One block: pack, bitonic sort in LDS, resolve by binary search in LDS, write table.
template <typename K>
__global__ __launch_bounds__(1024) void k_build_small(const int4 *__restrict__ coords, int n,
                                                      int res, int batch, int rb,
                                                      K *__restrict__ keys_out,
                                                      int32_t *__restrict__ perm_out,
                                                      int32_t *__restrict__ nbr, DevStatus *st)
{
    __shared__ K s_key[SMALL_N];
    __shared__ int32_t s_row[SMALL_N];
    __shared__ uint32_t s_red[1];
    const int tid = threadIdx.x;
    int np = 1;
    while (np < n) np <<= 1;
    bool bad_any = false;
    for (int i = tid; i < np; i += 1024) {
        if (i < n) {
            const int4 c = coords[i];
            const bool bad = (unsigned)c.x >= (unsigned)batch || (unsigned)c.y >= (unsigned)res ||
                             (unsigned)c.z >= (unsigned)res || (unsigned)c.w >= (unsigned)res;
            bad_any |= bad;
            s_key[i] = bad ? K(0) : pack_key<K>(c.x, c.y, c.z, c.w, rb);
            s_row[i] = i;
        } else {
            s_key[i] = (K)~K(0);  // padding sorts last: largest key, then largest row
            s_row[i] = 0x7fffffff;
        }
    }
    if (tid == 0) s_red[0] = 0;
    if (bad_any) atomicOr(&st->flags, FLAG_RANGE);
    __syncthreads();
    // bitonic sort of (key, row) pairs, ordered by key then row, so that padding
    // (all-ones key, largest row) lands behind every real entry even when a real
    // key is all ones
    for (int size = 2; size <= np; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < np; i += 1024) {
                const int j = i ^ stride;
                if (j > i) {
                    const bool up = (i & size) == 0;
                    const K a = s_key[i], b = s_key[j];
                    const bool greater = a > b || (a == b && s_row[i] > s_row[j]);
                    if (greater == up) {
                        s_key[i] = b;
                        s_key[j] = a;
                        const int32_t t = s_row[i];
                        s_row[i] = s_row[j];
                        s_row[j] = t;
                    }
                }
            }
            __syncthreads();
        }
    }
    const K m = (K(1) << rb) - 1;
    uint32_t present = 0;
    for (int s = tid; s < n; s += 1024) {
        const K key = s_key[s];
        keys_out[s] = key;
        perm_out[s] = s_row[s];
        if (s + 1 < n && s_key[s + 1] == key) atomicOr(&st->flags, FLAG_DUPLICATE);
        const int x = (int)(key & m), y = (int)((key >> rb) & m), z = (int)((key >> (2 * rb)) & m);
        const K bpart = (key >> (3 * rb)) << (3 * rb);
        int32_t *out = nbr + (int64_t)s_row[s] * 27;
        for (int k = 0; k < 27; ++k) {
            const int nz = z + k / 9 - 1, ny = y + (k / 3) % 3 - 1, nx = x + k % 3 - 1;
            int32_t r = -1;
            if (nz >= 0 && nz < res && ny >= 0 && ny < res && nx >= 0 && nx < res) {
                const K t = bpart | ((K)nz << (2 * rb)) | ((K)ny << rb) | (K)nx;
                const int64_t p = lower_bound_key(s_key, n, t);
                if (p < n && s_key[p] == t) r = s_row[p];
            }
            present += r >= 0;
            out[k] = r;
        }
    }
    if (present) atomicAdd(&s_red[0], present);
    __syncthreads();
    if (tid == 0 && s_red[0]) atomicAdd(&st->taps, (unsigned long long)s_red[0]);
}

// ---------------------------------------------------------------------------
// dense key space: occupancy bitmap + rank
// ---------------------------------------------------------------------------

template <typename K>
__global__ __launch_bounds__(256) void k_mark(const int4 *__restrict__ coords, int64_t n, int res,
                                              int batch, int rb, K *__restrict__ keys,
                                              unsigned long long *__restrict__ bm, DevStatus *st)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const unsigned lane = threadIdx.x & 63;
    bool valid = i < n, bad = false;
    K key = K(0);
    if (valid) {
        const int4 c = coords[i];
        bad = (unsigned)c.x >= (unsigned)batch || (unsigned)c.y >= (unsigned)res ||
              (unsigned)c.z >= (unsigned)res || (unsigned)c.w >= (unsigned)res;
        if (!bad) key = pack_key<K>(c.x, c.y, c.z, c.w, rb);
        keys[i] = key;
    }
    if (bad) atomicOr(&st->flags, FLAG_RANGE);
    const bool live = valid && !bad;
    // Runs of consecutive lanes that set bits of the same word (ordered inputs) are
    // merged by a segmented inclusive OR-scan (head flag = first lane of a run), so
    // only the last lane of each run touches memory.  Two lanes of one run with the
    // same bit are a duplicate; each merge joins disjoint lane ranges, so checking
    // the overlap at every merge sees every such pair.
    const uint64_t word = live ? (uint64_t)(key >> 6) : ~uint64_t(0);
    const unsigned long long bit = live ? (1ull << (uint32_t)(key & 63)) : 0ull;
    const uint64_t w_prev = __shfl_up(word, 1, 64);
    bool head = lane == 0 || w_prev != word;
    unsigned long long acc = bit;
    bool dup_in_run = false;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const unsigned long long a_up = __shfl_up(acc, off, 64);
        const bool h_up = __shfl_up((int)head, off, 64) != 0;
        if (lane >= (unsigned)off && !head) {
            dup_in_run |= (a_up & acc) != 0ull;
            acc |= a_up;
            head = h_up;
        }
    }
    const uint64_t w_next = __shfl_down(word, 1, 64);
    const bool last_of_run = lane == 63 || w_next != word;
    if (live && last_of_run) {
        const unsigned long long old = atomicOr(&bm[word], acc);
        if (old & acc) dup_in_run = true;
    }
    if (live && dup_in_run) atomicOr(&st->flags, FLAG_DUPLICATE);
}

template <typename K>
__device__ __forceinline__ int64_t rank_of(K key, const unsigned long long *bm, const uint32_t *prefix)
{
    const unsigned long long word = bm[key >> 6];
    return (int64_t)prefix[key >> 6] + __popcll(word & ((1ull << (uint32_t)(key & 63)) - 1ull));
}

template <typename K>
__global__ __launch_bounds__(256) void k_rank(const K *__restrict__ keys, int64_t n,
                                              const unsigned long long *__restrict__ bm,
                                              const uint32_t *__restrict__ prefix,
                                              K *__restrict__ sk, int32_t *__restrict__ perm)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const K key = keys[i];
    const int64_t r = rank_of(key, bm, prefix);
    if (r < n) {  // always, unless the set is invalid (then the build reports an error)
        sk[r] = key;
        perm[r] = (int32_t)i;
    }
}

template <typename K>
__global__ __launch_bounds__(256) void k_resolve_bm(const K *__restrict__ keys, int64_t n, int res,
                                                    int rb, const unsigned long long *__restrict__ bm,
                                                    const uint32_t *__restrict__ prefix,
                                                    const int32_t *__restrict__ perm,
                                                    int32_t *__restrict__ nbr, DevStatus *st)
{
    __shared__ int32_t s_rows[256 * 27];
    __shared__ uint32_t s_red[4];
    const int tid = threadIdx.x;
    const int64_t i0 = (int64_t)blockIdx.x * 256;
    const int count = (int)((n - i0) < 256 ? (n - i0) : 256);
    uint32_t present = 0;
    if (tid < count) {
        const K key = keys[i0 + tid];
        const K m = (K(1) << rb) - 1;
        const int x = (int)(key & m), y = (int)((key >> rb) & m), z = (int)((key >> (2 * rb)) & m);
        const K bpart = (key >> (3 * rb)) << (3 * rb);
        int32_t *row = s_rows + tid * 27;
        // ranks first (bitmap + prefix), then the rows at those ranks: 27 independent chains
        int64_t p[27];
#pragma unroll
        for (int d = 0; d < 9; ++d) {
            const int dz = d / 3 - 1, dy = d % 3 - 1;
            const int nz = z + dz, ny = y + dy;
            const bool row_ok = nz >= 0 && nz < res && ny >= 0 && ny < res;
            const K rowkey = bpart | ((K)nz << (2 * rb)) | ((K)ny << rb);
#pragma unroll
            for (int dx = -1; dx <= 1; ++dx) {
                const int nx = x + dx;
                p[3 * d + dx + 1] = -1;
                if (row_ok && nx >= 0 && nx < res) {
                    const K t = rowkey | (K)nx;
                    const unsigned long long word = bm[t >> 6];
                    const uint32_t b = (uint32_t)(t & 63);
                    if ((word >> b) & 1ull)
                        p[3 * d + dx + 1] = (int64_t)prefix[t >> 6] + __popcll(word & ((1ull << b) - 1ull));
                }
            }
        }
#pragma unroll
        for (int k = 0; k < 27; ++k) {
            const int32_t r = (p[k] >= 0 && p[k] < n) ? perm[p[k]] : -1;
            row[k] = r;
            present += r >= 0;
        }
    }
    uint32_t total;
    block_incl_scan256(present, s_red, &total);  // also the barrier for s_rows
    if (tid == 0 && total) atomicAdd(&st->taps, (unsigned long long)total);
    int32_t *dst = nbr + i0 * 27;  // rows i0 .. i0+count-1 are contiguous
    for (int e = tid; e < count * 27; e += 256) dst[e] = s_rows[e];
}

// One block, key space of at most 2^16 bits: the bitmap, its prefix and the
// sorted rows all live in LDS.
constexpr int SMALL_BITS = 16;

template <typename K>
__global__ __launch_bounds__(1024) void k_build_small_bm(const int4 *__restrict__ coords, int n,
                                                         int res, int batch, int rb, int nbits,
                                                         K *__restrict__ keys_out,
                                                         int32_t *__restrict__ perm_out,
                                                         int32_t *__restrict__ nbr, DevStatus *st)
{
    constexpr int WORDS = (1 << SMALL_BITS) / 32;
    __shared__ uint32_t s_bm[WORDS];
    __shared__ uint32_t s_pre[WORDS];
    __shared__ int32_t s_perm[SMALL_N];
    __shared__ uint32_t s_wave[16];
    __shared__ uint32_t s_flags, s_taps;
    const int tid = threadIdx.x;
    const int words = nbits > 5 ? (1 << (nbits - 5)) : 1;
    for (int w = tid; w < words; w += 1024) s_bm[w] = 0;
    if (tid == 0) { s_flags = 0; s_taps = 0; }
    __syncthreads();
    K key[2];
    bool ok[2];
    for (int q = 0; q < 2; ++q) {  // n <= 2048 = 2 per thread
        const int i = tid + q * 1024;
        ok[q] = false;
        key[q] = K(0);
        if (i < n) {
            const int4 c = coords[i];
            const bool bad = (unsigned)c.x >= (unsigned)batch || (unsigned)c.y >= (unsigned)res ||
                             (unsigned)c.z >= (unsigned)res || (unsigned)c.w >= (unsigned)res;
            if (bad) atomicOr(&s_flags, FLAG_RANGE);
            else {
                key[q] = pack_key<K>(c.x, c.y, c.z, c.w, rb);
                ok[q] = true;
                const uint32_t bit = 1u << (uint32_t)(key[q] & 31);
                if (atomicOr(&s_bm[key[q] >> 5], bit) & bit) atomicOr(&s_flags, FLAG_DUPLICATE);
            }
        }
    }
    __syncthreads();
    // exclusive prefix of word popcounts (words <= 2048: two per thread)
    {
        const int w0 = 2 * tid;
        const uint32_t a = w0 < words ? (uint32_t)__popc(s_bm[w0]) : 0u;
        const uint32_t b = w0 + 1 < words ? (uint32_t)__popc(s_bm[w0 + 1]) : 0u;
        const uint32_t v = a + b;
        const unsigned lane = tid & 63, wave = tid >> 6;
        uint32_t x = v;
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(x, off, 64);
            if (lane >= (unsigned)off) x += y;
        }
        if (lane == 63) s_wave[wave] = x;
        __syncthreads();
        uint32_t before = 0;
        for (int w = 0; w < (int)wave; ++w) before += s_wave[w];
        const uint32_t ex = x - v + before;
        if (w0 < words) s_pre[w0] = ex;
        if (w0 + 1 < words) s_pre[w0 + 1] = ex + a;
    }
    __syncthreads();
    if (s_flags) {  // invalid set: report only
        if (tid == 0) atomicOr(&st->flags, s_flags);
        return;
    }
    for (int q = 0; q < 2; ++q) {
        const int i = tid + q * 1024;
        if (ok[q]) {
            const int r = (int)(s_pre[key[q] >> 5] + __popc(s_bm[key[q] >> 5] & ((1u << (uint32_t)(key[q] & 31)) - 1u)));
            s_perm[r] = i;
            keys_out[r] = key[q];
            perm_out[r] = i;
        }
    }
    __syncthreads();
    const K m = (K(1) << rb) - 1;
    uint32_t present = 0;
    for (int q = 0; q < 2; ++q) {
        const int i = tid + q * 1024;
        if (!ok[q]) continue;
        const int x = (int)(key[q] & m), y = (int)((key[q] >> rb) & m), z = (int)((key[q] >> (2 * rb)) & m);
        const K bpart = (key[q] >> (3 * rb)) << (3 * rb);
        int32_t *out = nbr + (int64_t)i * 27;
        for (int k = 0; k < 27; ++k) {
            const int nz = z + k / 9 - 1, ny = y + (k / 3) % 3 - 1, nx = x + k % 3 - 1;
            int32_t r = -1;
            if (nz >= 0 && nz < res && ny >= 0 && ny < res && nx >= 0 && nx < res) {
                const K t = bpart | ((K)nz << (2 * rb)) | ((K)ny << rb) | (K)nx;
                const uint32_t word = s_bm[t >> 5], b = (uint32_t)(t & 31);
                if ((word >> b) & 1u) r = s_perm[s_pre[t >> 5] + __popc(word & ((1u << b) - 1u))];
            }
            present += r >= 0;
            out[k] = r;
        }
    }
    if (present) atomicAdd(&s_taps, present);
    __syncthreads();
    if (tid == 0 && s_taps) atomicAdd(&st->taps, (unsigned long long)s_taps);
}

// Bitmap bytes are affordable when they stay within a small multiple of the
// per-voxel data (a 512^3 grid of 3M voxels: 16 MB).
static bool use_bitmap(int64_t n, int nbits)
{
    if (nbits > 31) return false;
    const int64_t bytes = (int64_t(1) << nbits) / 8;
    return bytes <= 64 * n + (int64_t(4) << 20);
}

template <typename K>
static int build_map_impl(const int32_t *coords, submconv_rulebook *rb, hipStream_t stream)
{
    const int64_t n = rb->n;
    const int path = (n <= SMALL_N && rb->nbits <= SMALL_BITS) ? 0 : (n <= SMALL_N ? 1 : (use_bitmap(n, rb->nbits) ? 2 : 3));
    auto up = [](size_t b) { return (b + 255) & ~size_t(255); };
    const int64_t words = rb->nbits > 6 ? (int64_t(1) << (rb->nbits - 6)) : 1;  // 64-bit bitmap words
    // scratch: path 2 = tmp keys, bitmap, prefix, scan scratch; path 3 = alt keys/rows, sort scratch
    size_t off = 0, o_keys = 0, o_vals = 0, o_bm = 0, o_pre = 0, o_aux = 0;
    if (path == 2) {
        o_keys = off; off += up((size_t)n * sizeof(K));
        o_bm = off; off += up((size_t)words * 8);
        o_pre = off; off += up((size_t)words * 4);
        o_aux = off; off += up(scan_scratch_bytes(words));
    } else if (path == 3) {
        o_keys = off; off += up((size_t)n * sizeof(K));
        o_vals = off; off += up((size_t)n * 4);
        o_aux = off; off += up(sort_scratch_bytes(n));
    }
    const size_t o_stat = off;
    off += sizeof(DevStatus);
    char *scratch = nullptr;
    SC_CHECK(dev_alloc((void **)&scratch, off, stream));
    DevStatus *st = (DevStatus *)(scratch + o_stat);
    int status = SUBMCONV_OK;
    const unsigned grid = (unsigned)((n + 255) / 256);
    do {
        if (hipMemsetAsync(st, 0, sizeof(DevStatus), stream) != hipSuccess) { status = fail(SUBMCONV_E_HIP, "status clear failed"); break; }
        if (path == 0) {
            hipLaunchKernelGGL(k_build_small_bm<K>, dim3(1), dim3(1024), 0, stream, (const int4 *)coords,
                               (int)n, rb->res, rb->batch, rb->rb, rb->nbits, (K *)rb->keys, rb->perm, rb->nbr, st);
        } else if (path == 1) {
            hipLaunchKernelGGL(k_build_small<K>, dim3(1), dim3(1024), 0, stream, (const int4 *)coords,
                               (int)n, rb->res, rb->batch, rb->rb, (K *)rb->keys, rb->perm, rb->nbr, st);
        } else if (path == 2) {
            K *tmp = (K *)(scratch + o_keys);
            unsigned long long *bm = (unsigned long long *)(scratch + o_bm);
            uint32_t *pre = (uint32_t *)(scratch + o_pre);
            if (hipMemsetAsync(bm, 0, (size_t)words * 8, stream) != hipSuccess) { status = fail(SUBMCONV_E_HIP, "bitmap clear failed"); break; }
            hipLaunchKernelGGL(k_mark<K>, dim3(grid), dim3(256), 0, stream, (const int4 *)coords, n, rb->res,
                               rb->batch, rb->rb, tmp, bm, st);
            if ((status = exclusive_scan_u32((const uint32_t *)bm, pre, words, nullptr, scratch + o_aux, stream, SCAN_POPC64)) != SUBMCONV_OK) break;
            hipLaunchKernelGGL(k_rank<K>, dim3(grid), dim3(256), 0, stream, (const K *)tmp, n, bm, pre,
                               (K *)rb->keys, rb->perm);
            hipLaunchKernelGGL(k_resolve_bm<K>, dim3(grid), dim3(256), 0, stream, (const K *)tmp, n, rb->res,
                               rb->rb, bm, pre, rb->perm, rb->nbr, st);
        } else {
            K *keys_b = (K *)(scratch + o_keys);
            int32_t *vals_b = (int32_t *)(scratch + o_vals);
            const bool in_b = radix_sort_passes(n, rb->nbits) & 1;  // lands in rb->keys without a copy
            hipLaunchKernelGGL(k_pack<K>, dim3(grid), dim3(256), 0, stream, (const int4 *)coords, n,
                               rb->res, rb->batch, rb->rb, in_b ? keys_b : (K *)rb->keys,
                               in_b ? vals_b : rb->perm, st);
            if ((status = radix_sort_pairs<K>((K *)rb->keys, rb->perm, keys_b, vals_b, n, rb->nbits,
                                              scratch + o_aux, stream, in_b)) != SUBMCONV_OK) break;
            hipLaunchKernelGGL(k_resolve_win<K>, dim3(grid), dim3(256), 0, stream, (const K *)rb->keys,
                               rb->perm, n, rb->res, rb->rb, rb->nbr, st);
        }
        if (hipGetLastError() != hipSuccess) { status = fail(SUBMCONV_E_HIP, "kernel launch in build_map failed"); break; }
        DevStatus h;
        if ((status = read_status(st, &h, stream)) != SUBMCONV_OK) break;
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
