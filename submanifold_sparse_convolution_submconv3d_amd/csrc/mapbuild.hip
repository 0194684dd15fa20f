// Neighbour-map ("rulebook") builder for the submanifold 3x3x3 convolution.
//
// The pages resolve neighbours through a sorted key array with 27 lookups per
// voxel, cached per coordinate set (lato.2_mrp_mlx working notes, commit
// summary).  Every coordinate is validated and packed into an integer key
// ((b << 3rb) | (z << 2rb) | (y << rb) | x); keys are sorted, and each voxel's
// 27 neighbour keys are looked up in the sorted order.
//
// What the rulebook keeps, all indexed by sorted position s (C order of
// (b, z, y, x)):
//   keys[s], perm[s] (the input row of sorted voxel s),
//   nbr_sp[s]     the SORTED POSITIONS of the voxels at key[s] + offset(k), in the
//                 row form of NBR_INTS ints (common.h): per (dz, dy) row the first
//                 present position and presence bits, 40 bytes instead of 108,
//   gwin[g]        per group of 32 consecutive sorted voxels and per (dz, dy)
//                  row: the first and last sorted position the group's
//                  neighbours in that row occupy.  A kernel merges the windows
//                  of the groups it processes into a few ranges of sorted
//                  positions, stages them in LDS and indexes them directly.
// The input-order table nbr[i][k] (input rows) is derived from these on request.
//
// Dense key space (2^nbits bitmap bits affordable next to N):
//   mark     - set the key's bit in an occupancy bitmap (no-return atomicOr;
//              lanes of a wave that hit the same word are combined first);
//   scan     - exclusive scan of the bitmap words' popcounts; its total is the
//              number of distinct keys, so a total below N means a duplicate;
//   rank     - a key's sorted position is prefix[word] + popcount of the lower
//              bits of its word: one radix pass whose digit is the whole key
//              (histogram = bitmap, counts are 0/1 because keys are distinct);
//   resolve  - per sorted voxel, each neighbour is a bit test plus the same rank
//              query; no gathers, and table rows are written as coalesced runs.
// Sparse key space (huge grid, few voxels):
//   pack + multi-pass LSD radix sort, then per tile of 256 sorted voxels: the x
//   neighbours of the centre row are the adjacent sorted entries; for each of the
//   other 8 (dz, dy) rows every target key lies in [first + off - 1, last + off + 1]
//   (off = the row's key offset), so the block copies that window of sorted keys
//   into LDS and binary-searches there (a window too big for LDS is searched in
//   place).
// Small sets (n <= 2048) build in one block.  Coordinates are range-checked
// before packing and every neighbour coordinate is bounds-checked before its key
// is formed, so a key never wraps into the next row, plane or batch entry.
#include "common.h"

namespace sc {

constexpr int WIN_MAX = 2048;      // window keys held in LDS (sparse path)
constexpr int SMALL_N = 2048;      // single-block build up to this many voxels
constexpr int SMALL_BITS = 16;     // single-block bitmap up to 2^16 bits

template <typename K>
__device__ __forceinline__ K pack_key(int b, int z, int y, int x, int rb)
{
    return ((((K)b << rb | (K)z) << rb | (K)y) << rb) | (K)x;
}

template <typename K>
__device__ __forceinline__ bool key_valid(K key, int rb, int res, int batch)
{
    const K m = (K(1) << rb) - 1;
    return (uint64_t)(key >> (3 * rb)) < (uint64_t)batch && (int)(key & m) < res &&
           (int)((key >> rb) & m) < res && (int)((key >> (2 * rb)) & m) < res;
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

// ---------------------------------------------------------------------------
// group windows
// ---------------------------------------------------------------------------

// Write the row windows of the wave's two groups (lanes 0-31, 32-63) from each
// lane's 27 sorted positions.  Every lane of the wave must call it, lanes in
// sorted order; groups at or past `ngroups` are not written.
//
// For a fixed (dz, dy) row the window [first present, last present] of a voxel
// is monotone in sorted order: a later voxel's cells are all >= the earlier
// voxel's cell at dx = 0, which is present or else not before the earlier
// voxel's first present cell.  So a group's window for the row is the first
// such lane's lo and the last such lane's hi: one ballot per row, no reduction.
__device__ __forceinline__ void group_windows_write(const int32_t (&p)[27], bool valid, int64_t group,
                                                    int64_t ngroups, int32_t *__restrict__ gwin)
{
    const int lane = (int)(threadIdx.x & 63), half = lane >> 5;
    const bool owner = group < ngroups;
    int32_t *w = gwin + group * GWIN_INTS;
#pragma unroll
    for (int d = 0; d < 9; ++d) {
        const int32_t a = p[3 * d], b = p[3 * d + 1], c = p[3 * d + 2];
        const int32_t lo = a >= 0 ? a : (b >= 0 ? b : c);
        const int32_t hi = c >= 0 ? c : (b >= 0 ? b : a);
        const uint64_t mask = __ballot(valid && hi >= 0);
        const uint32_t m = (uint32_t)(mask >> (32 * half));
        const int first = m ? __ffs((int)m) - 1 : 0;
        const int last = m ? 31 - __clz((int)m) : 0;
        if (owner && (lane & 31) == first) w[d] = m ? lo : GWIN_NONE;
        if (owner && (lane & 31) == last) w[9 + d] = m ? hi : -1;
    }
}

// The same from a packed neighbour row (first positions and presence bits).
__device__ __forceinline__ void group_windows_write_row(const int32_t (&r)[NBR_INTS], bool valid, int64_t group,
                                                        int64_t ngroups, int32_t *__restrict__ gwin)
{
    const int lane = (int)(threadIdx.x & 63), half = lane >> 5;
    const bool owner = group < ngroups;
    int32_t *w = gwin + group * GWIN_INTS;
#pragma unroll
    for (int d = 0; d < 9; ++d) {
        const uint32_t bits = ((uint32_t)r[9] >> (3 * d)) & 7u;
        const uint64_t mask = __ballot(valid && bits != 0u);
        const uint32_t m = (uint32_t)(mask >> (32 * half));
        const int first = m ? __ffs((int)m) - 1 : 0;
        const int last = m ? 31 - __clz((int)m) : 0;
        if (owner && (lane & 31) == first) w[d] = m ? r[d] : GWIN_NONE;
        if (owner && (lane & 31) == last) w[9 + d] = m ? r[d] + (int32_t)__popc(bits) - 1 : -1;
    }
}

// Table rows of one block from LDS to global (a contiguous run) and the block's
// present count.  Called by every thread after its row of s_rows is written and
// its count is added to *s_taps.
__device__ __forceinline__ void block_finish(const int32_t *s_rows, int count, int32_t *dst,
                                             const uint32_t *s_taps, uint32_t *blk_taps)
{
    __syncthreads();
    if (threadIdx.x == 0) blk_taps[blockIdx.x] = *s_taps;
    for (int e = threadIdx.x; e < count * NBR_INTS; e += 256) dst[e] = s_rows[e];
}

// ---------------------------------------------------------------------------
// dense key space: occupancy bitmap + rank
// ---------------------------------------------------------------------------

constexpr int MARK_ROWS = 4;        // rows per thread in k_mark
constexpr int MARK_SLOTS = 2048;    // LDS hash slots per block (2 x the block's rows)
constexpr unsigned long long MARK_EMPTY = ~0ull;

// Validate and pack each row's key, and set its bit in the occupancy bitmap.  A
// block first ORs its rows' bits into an LDS hash table keyed by bitmap word, so
// each distinct word costs one device-scope atomic per block instead of one per
// row (device-scope atomics execute at the memory side on this chip).  Ordered
// inputs touch few words per block.
template <typename K>
__global__ __launch_bounds__(256) void k_mark(const int4 *__restrict__ coords, int64_t n, int res,
                                              int batch, int rb, K *__restrict__ keys,
                                              unsigned long long *__restrict__ bm, DevStatus *st)
{
    __shared__ unsigned long long s_word[MARK_SLOTS], s_bits[MARK_SLOTS];
    for (int i = threadIdx.x; i < MARK_SLOTS; i += 256) {
        s_word[i] = MARK_EMPTY;
        s_bits[i] = 0ull;
    }
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * (256 * MARK_ROWS) + threadIdx.x;
    bool bad_any = false;
    // all rows' loads first (clamped index, no branch), so they share one round trip
    int4 cq[MARK_ROWS];
#pragma unroll
    for (int q = 0; q < MARK_ROWS; ++q) {
        const int64_t i = base + q * 256;  // consecutive threads read consecutive rows
        cq[q] = coords[i < n ? i : n - 1];
    }
#pragma unroll
    for (int q = 0; q < MARK_ROWS; ++q) {
        const int64_t i = base + q * 256;
        if (i >= n) continue;
        const int4 c = cq[q];
        const bool bad = (unsigned)c.x >= (unsigned)batch || (unsigned)c.y >= (unsigned)res ||
                         (unsigned)c.z >= (unsigned)res || (unsigned)c.w >= (unsigned)res;
        bad_any |= bad;
        K key = (K)~K(0);  // marks an invalid row for the rank pass
        if (!bad) {
            key = pack_key<K>(c.x, c.y, c.z, c.w, rb);
            const unsigned long long w = (unsigned long long)(key >> 6);
            uint32_t h = ((uint32_t)w * 0x9E3779B1u) >> (32 - 11);
            // linear probing; the table has twice the block's rows, so it never fills
            for (;;) {
                const unsigned long long prev = atomicCAS(&s_word[h], MARK_EMPTY, w);
                if (prev == MARK_EMPTY || prev == w) break;
                h = (h + 1) & (MARK_SLOTS - 1);
            }
            atomicOr(&s_bits[h], 1ull << (uint32_t)(key & 63));
        }
        keys[i] = key;
    }
    if (bad_any) atomicOr(&st->flags, FLAG_RANGE);
    __syncthreads();
    for (int i = threadIdx.x; i < MARK_SLOTS; i += 256) {
        const unsigned long long w = s_word[i];
        if (w != MARK_EMPTY) atomicOr(&bm[w], s_bits[i]);
    }
}

template <typename K>
__global__ __launch_bounds__(256) void k_rank(const K *__restrict__ keys, int64_t n,
                                              const unsigned long long *__restrict__ bm,
                                              const uint32_t *__restrict__ prefix,
                                              const uint32_t *__restrict__ tsum,
                                              K *__restrict__ sk, int32_t *__restrict__ perm)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const K key = keys[i];
    if (key == (K)~K(0)) return;  // out-of-range row (the build reports it)
    const unsigned long long word = bm[key >> 6];
    const uint64_t w = (uint64_t)(key >> 6);
    const int64_t r = (int64_t)prefix[w] + tsum[w / SCAN_TILE_ITEMS] +
                      __popcll(word & ((1ull << (uint32_t)(key & 63)) - 1ull));
    if (r < n) {
        sk[r] = key;
        perm[r] = (int32_t)i;
    }
}

template <typename K>
__global__ __launch_bounds__(256) void k_resolve_bm(const K *__restrict__ sk, int64_t n, int res, int rb,
                                                    int batch, const unsigned long long *__restrict__ bm,
                                                    const uint32_t *__restrict__ prefix,
                                                    const uint32_t *__restrict__ tsum,
                                                    int32_t *__restrict__ nbr_sp,
                                                    int32_t *__restrict__ gwin,
                                                    uint32_t *__restrict__ blk_taps)
{
    __shared__ int32_t s_rows[256 * NBR_INTS];
    __shared__ uint32_t s_taps;
    const int tid = threadIdx.x;
    const int64_t s0 = (int64_t)blockIdx.x * 256;
    const int count = (int)((n - s0) < 256 ? (n - s0) : 256);
    if (tid == 0) s_taps = 0;
    __syncthreads();
    // the packed row (first position per (dz, dy) row, presence bits), built
    // straight from each row's three occupancy bits and the rank of its first cell
    int32_t r[NBR_INTS];
#pragma unroll
    for (int q = 0; q < NBR_INTS; ++q) r[q] = 0;
    uint32_t present = 0;
    K key = K(0);
    if (tid < count) key = sk[s0 + tid];
    // positions past the last distinct key are never written when the set holds
    // a duplicate or an invalid row (the build then reports an error): skip them
    const bool valid = tid < count && key_valid(key, rb, res, batch);
    if (valid) {
        const uint32_t s = (uint32_t)(s0 + tid), un = (uint32_t)n;  // positions fit in 31 bits
        const K m = (K(1) << rb) - 1;
        const int x = (int)(key & m), y = (int)((key >> rb) & m), z = (int)((key >> (2 * rb)) & m);
        const K bpart = (key >> (3 * rb)) << (3 * rb);
        const int xs = x > 0 ? x - 1 : 0;                      // first cell of each row window
        const uint32_t valid3 = (x > 0 ? 1u : 0u) | 2u | (x + 1 < res ? 4u : 0u);  // cells x-1, x, x+1 on the grid
        const uint32_t shift = x > 0 ? 0u : 1u;                // window bit j <-> cell x-1+j
        // Each row (dz, dy): the occupancy of cells x-1 .. x+1 (3 bits, from one or
        // two words) and the rank of the row's first cell; the present cells take
        // consecutive positions from there.  All loads are issued without branching
        // (rows off the grid read word 0 and are masked), so the whole neighbourhood
        // costs one memory round trip.
        K wd[9];
        uint32_t bsh[9];
        bool rok[9];
#pragma unroll
        for (int d = 0; d < 9; ++d) {
            const int nz = z + d / 3 - 1, ny = y + d % 3 - 1;
            rok[d] = nz >= 0 && nz < res && ny >= 0 && ny < res;
            const K c0 = rok[d] ? (K)(bpart | ((K)nz << (2 * rb)) | ((K)ny << rb) | (K)xs) : K(0);
            wd[d] = c0 >> 6;
            bsh[d] = (uint32_t)(c0 & 63);
        }
        // Of the next word only the low two bits can fall in the window: load its low
        // half only (the bitmap has one word of padding).  A 64-bit load whose upper
        // half is dead lets the compiler reuse that register at once, which makes it
        // wait for the load there and serialises the round trips.
        unsigned long long lo_w[9];
        uint32_t hi_w[9], pre[9];
        const uint32_t *bm32 = (const uint32_t *)bm;
#pragma unroll
        for (int d = 0; d < 9; ++d) {
            lo_w[d] = bm[wd[d]];
            hi_w[d] = bm32[2 * wd[d] + 2];
            pre[d] = prefix[wd[d]] + tsum[wd[d] / SCAN_TILE_ITEMS];
        }
        uint32_t mask = 0;
#pragma unroll
        for (int d = 0; d < 9; ++d) {
            const uint32_t b = bsh[d];
            unsigned long long v = lo_w[d] >> b;
            if (b > 61) v |= (unsigned long long)hi_w[d] << (64 - b);
            uint32_t bits = rok[d] ? (((uint32_t)(v & 7ull) << shift) & valid3) : 0u;
            // keys below the row window's first cell (the centre row: the voxel is at s)
            const uint32_t q = (d == 4) ? s - (bits & 1u)
                                        : pre[d] + (uint32_t)__popcll(lo_w[d] & ((1ull << b) - 1ull));
            // a cell whose position would be n or more (a set with duplicates or
            // invalid rows, which the build reports) is dropped
            if (q + (uint32_t)__popc(bits) > un) {
                uint32_t keep = q < un ? un - q : 0u, kept = 0;
#pragma unroll
                for (int j = 0; j < 3; ++j)
                    if (((bits >> j) & 1u) && keep) { kept |= 1u << j; --keep; }
                bits = kept;
            }
            r[d] = bits ? (int32_t)q : 0;
            mask |= bits << (3 * d);
        }
        r[9] = (int32_t)mask;
        present = (uint32_t)__popc(mask);
    }
    if (tid < count) {
#pragma unroll
        for (int q = 0; q < NBR_INTS; ++q) s_rows[tid * NBR_INTS + q] = r[q];
    }
    if (present) atomicAdd(&s_taps, present);
    group_windows_write_row(r, valid, (s0 + tid) >> 5, (n + 31) >> 5, gwin);
    block_finish(s_rows, count, nbr_sp + s0 * NBR_INTS, &s_taps, blk_taps);
}

// ---------------------------------------------------------------------------
// sparse key space: radix sort + windowed search
// ---------------------------------------------------------------------------

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

template <typename K>
__global__ __launch_bounds__(256) void k_resolve_win(const K *__restrict__ sk, int64_t n, int res,
                                                     int rb, int32_t *__restrict__ nbr_sp,
                                                     int32_t *__restrict__ gwin,
                                                     uint32_t *__restrict__ blk_taps, DevStatus *st)
{
    __shared__ K s_win[WIN_MAX];
    __shared__ int32_t s_rows[256 * NBR_INTS];
    __shared__ int64_t s_wlo[8], s_whi[8];
    __shared__ uint32_t s_taps;

    const int tid = threadIdx.x;
    const int64_t s0 = (int64_t)blockIdx.x * 256;
    const int count = (int)((n - s0) < 256 ? (n - s0) : 256);
    const int64_t s = s0 + tid;
    const bool valid = tid < count;
    const K m = (K(1) << rb) - 1;
    const K key = valid ? sk[s] : K(0);
    const int x = (int)(key & m), y = (int)((key >> rb) & m), z = (int)((key >> (2 * rb)) & m);
    const K bpart = (key >> (3 * rb)) << (3 * rb);
    if (tid == 0) s_taps = 0;
    // window bounds of the 8 off-centre (dz, dy) rows: 16 binary searches, one per thread
    if (tid < 16) {
        int d = tid >> 1;
        d += (d >= 4);  // skip the centre row (dz, dy) = (0, 0)
        const int dz = d / 3 - 1, dy = d % 3 - 1;
        const int64_t off = (int64_t)dz * ((int64_t)1 << (2 * rb)) + (int64_t)dy * ((int64_t)1 << rb);
        const K first = sk[s0], last = sk[s0 + count - 1];
        int64_t r;
        if ((tid & 1) == 0) r = lower_bound_key(sk, n, add_sat(first, off - 1));
        else {
            const K t = add_sat(last, off + 1);  // first index with a key > t
            r = (t == (K)~K(0)) ? n : lower_bound_key(sk, n, (K)(t + 1));
        }
        if ((tid & 1) == 0) s_wlo[tid >> 1] = r;
        else s_whi[tid >> 1] = r;
    }
    int32_t p[27];
#pragma unroll
    for (int k = 0; k < 27; ++k) p[k] = -1;
    bool dup = false;
    if (valid) {  // centre row: adjacent sorted entries
        dup = (s + 1 < n) && sk[s + 1] == key;
        if (x > 0 && s > 0 && sk[s - 1] == key - 1) p[12] = (int32_t)(s - 1);
        p[13] = (int32_t)s;
        if (x + 1 < res && s + 1 < n && sk[s + 1] == key + 1) p[14] = (int32_t)(s + 1);
    }
    __syncthreads();
    for (int w = 0; w < 8; ++w) {
        const int d = w + (w >= 4);
        const int dz = d / 3 - 1, dy = d % 3 - 1;
        const int64_t lo = s_wlo[w], hi = s_whi[w];
        const int64_t wn = hi - lo;
        const bool in_lds = wn <= WIN_MAX;
        if (in_lds)
            for (int i = tid; i < wn; i += 256) s_win[i] = sk[lo + i];
        __syncthreads();
        if (valid) {
            const int nz = z + dz, ny = y + dy;
            if (nz >= 0 && nz < res && ny >= 0 && ny < res) {
                const K rowkey = bpart | ((K)nz << (2 * rb)) | ((K)ny << rb);
                const K t0 = rowkey | (K)(x > 0 ? x - 1 : 0);
                int64_t q = in_lds ? lower_bound_key(s_win, wn, t0) : lower_bound_key(sk + lo, wn, t0);
                for (int dx = -1; dx <= 1; ++dx) {
                    const int nx = x + dx;
                    if (nx < 0 || nx >= res) continue;
                    const K t = rowkey | (K)nx;
                    if (in_lds) {
                        while (q < wn && s_win[q] < t) ++q;
                        if (q < wn && s_win[q] == t) p[3 * d + dx + 1] = (int32_t)(lo + q);
                    } else {
                        while (q < wn && sk[lo + q] < t) ++q;
                        if (q < wn && sk[lo + q] == t) p[3 * d + dx + 1] = (int32_t)(lo + q);
                    }
                }
            }
        }
        __syncthreads();
    }
    uint32_t present = 0;
    if (valid) {
        int32_t r[NBR_INTS];
        nbr_pack(p, r);
#pragma unroll
        for (int q = 0; q < NBR_INTS; ++q) s_rows[tid * NBR_INTS + q] = r[q];
#pragma unroll
        for (int k = 0; k < 27; ++k) present += p[k] >= 0;
    }
    if (dup) atomicOr(&st->flags, FLAG_DUPLICATE);
    if (present) atomicAdd(&s_taps, present);
    group_windows_write(p, valid, (s0 + tid) >> 5, (n + 31) >> 5, gwin);
    block_finish(s_rows, count, nbr_sp + s0 * NBR_INTS, &s_taps, blk_taps);
}

// ---------------------------------------------------------------------------
// small sets: one block
// ---------------------------------------------------------------------------

// Key space of at most 2^16 bits: bitmap and prefix in LDS.
template <typename K>
__global__ __launch_bounds__(1024) void k_build_small_bm(const int4 *__restrict__ coords, int n,
                                                         int res, int batch, int rb, int nbits,
                                                         K *__restrict__ keys_out,
                                                         int32_t *__restrict__ perm_out,
                                                         int32_t *__restrict__ nbr_sp, DevStatus *st)
{
    constexpr int WORDS = (1 << SMALL_BITS) / 32;
    __shared__ uint32_t s_bm[WORDS];
    __shared__ uint32_t s_pre[WORDS];
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
    {   // exclusive prefix of word popcounts (words <= 2048: two per thread)
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
    const K m = (K(1) << rb) - 1;
    uint32_t present = 0;
    for (int q = 0; q < 2; ++q) {
        if (!ok[q]) continue;
        const int i = tid + q * 1024;
        const int s = (int)(s_pre[key[q] >> 5] + __popc(s_bm[key[q] >> 5] & ((1u << (uint32_t)(key[q] & 31)) - 1u)));
        keys_out[s] = key[q];
        perm_out[s] = i;
        const int x = (int)(key[q] & m), y = (int)((key[q] >> rb) & m), z = (int)((key[q] >> (2 * rb)) & m);
        const K bpart = (key[q] >> (3 * rb)) << (3 * rb);
        int32_t p[27];
#pragma unroll
        for (int k = 0; k < 27; ++k) {
            const int nz = z + k / 9 - 1, ny = y + (k / 3) % 3 - 1, nx = x + k % 3 - 1;
            int32_t r = -1;
            if (nz >= 0 && nz < res && ny >= 0 && ny < res && nx >= 0 && nx < res) {
                const K t = bpart | ((K)nz << (2 * rb)) | ((K)ny << rb) | (K)nx;
                const uint32_t word = s_bm[t >> 5], b = (uint32_t)(t & 31);
                if ((word >> b) & 1u) r = (int32_t)(s_pre[t >> 5] + __popc(word & ((1u << b) - 1u)));
            }
            present += r >= 0;
            p[k] = r;
        }
        int32_t rr[NBR_INTS];
        nbr_pack(p, rr);
#pragma unroll
        for (int q = 0; q < NBR_INTS; ++q) nbr_sp[(int64_t)s * NBR_INTS + q] = rr[q];
    }
    if (present) atomicAdd(&s_taps, present);
    __syncthreads();
    if (tid == 0 && s_taps) atomicAdd(&st->taps, (unsigned long long)s_taps);
}

// Larger key space: bitonic sort of (key, row) in LDS, binary search in LDS.
template <typename K>
__global__ __launch_bounds__(1024) void k_build_small(const int4 *__restrict__ coords, int n,
                                                      int res, int batch, int rb,
                                                      K *__restrict__ keys_out,
                                                      int32_t *__restrict__ perm_out,
                                                      int32_t *__restrict__ nbr_sp, DevStatus *st)
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
        int32_t p[27];
#pragma unroll
        for (int k = 0; k < 27; ++k) {
            const int nz = z + k / 9 - 1, ny = y + (k / 3) % 3 - 1, nx = x + k % 3 - 1;
            int32_t r = -1;
            if (nz >= 0 && nz < res && ny >= 0 && ny < res && nx >= 0 && nx < res) {
                const K t = bpart | ((K)nz << (2 * rb)) | ((K)ny << rb) | (K)nx;
                const int64_t q = lower_bound_key(s_key, n, t);
                if (q < n && s_key[q] == t) r = (int32_t)q;
            }
            present += r >= 0;
            p[k] = r;
        }
        int32_t rr[NBR_INTS];
        nbr_pack(p, rr);
#pragma unroll
        for (int q = 0; q < NBR_INTS; ++q) nbr_sp[(int64_t)s * NBR_INTS + q] = rr[q];
    }
    if (present) atomicAdd(&s_red[0], present);
    __syncthreads();
    if (tid == 0 && s_red[0]) atomicAdd(&st->taps, (unsigned long long)s_red[0]);
}

// Group windows from a finished table (used after the single-block builds).
__global__ __launch_bounds__(256) void k_group_windows(const int32_t *__restrict__ nbr_sp, int64_t n,
                                                       int32_t *__restrict__ gwin)
{
    const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
    int32_t p[27];
    const bool valid = s < n;
#pragma unroll
    for (int k = 0; k < 27; ++k) p[k] = valid ? nbr_at(nbr_sp + s * NBR_INTS, k) : -1;
    group_windows_write(p, valid, s >> 5, (n + 31) >> 5, gwin);
}

// ---------------------------------------------------------------------------
// input-order table, on request
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_input_order_table(const int32_t *__restrict__ nbr_sp,
                                                           const int32_t *__restrict__ perm, int64_t n,
                                                           int32_t *__restrict__ out)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over n x 27, sorted order
    if (e >= n * 27) return;
    const int64_t s = e / 27;
    const int k = (int)(e - s * 27);
    const int32_t p = nbr_at(nbr_sp + s * NBR_INTS, k);
    const uint32_t row = (uint32_t)perm[s];
    if (row < (uint64_t)n) out[(int64_t)row * 27 + k] = (p >= 0 && p < n) ? perm[p] : -1;
}

int input_order_table(const submconv_rulebook *rb, int32_t *out, hipStream_t s)
{
    const int64_t total = rb->n * 27;
    if (total == 0) return SUBMCONV_OK;
    hipLaunchKernelGGL(k_input_order_table, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       rb->nbr_sp, rb->perm, rb->n, out);
    SC_LAUNCHED("input_order_table");
    return SUBMCONV_OK;
}

// ---------------------------------------------------------------------------
// driver
// ---------------------------------------------------------------------------

// Bitmap bytes are affordable when they stay within a small multiple of the
// per-voxel data (a 512^3 grid of 3M voxels: 16 MB).
int win_plan_build(submconv_rulebook *rb, const uint32_t *blk_taps, int64_t nblk, DevStatus *st,
                   hipStream_t s);  // conv_win.hip

// Zero the status block and `words` 64-bit words (the bitmap); grid-stride.
__global__ __launch_bounds__(256) void k_clear(DevStatus *st, unsigned long long *__restrict__ w, int64_t words)
{
    if (blockIdx.x == 0 && threadIdx.x == 0) *st = DevStatus{};
    // pairs of words as 16-byte stores (w is 16-byte aligned), then an odd last word
    const int64_t pairs = words >> 1;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < pairs; i += (int64_t)gridDim.x * 256)
        ((ulonglong2 *)w)[i] = make_ulonglong2(0ull, 0ull);
    if ((words & 1) && blockIdx.x == 0 && threadIdx.x == 0) w[words - 1] = 0ull;
}

static bool use_bitmap(int64_t n, int nbits)
{
    if (nbits > 31) return false;
    const int64_t bytes = (int64_t(1) << nbits) / 8;
    return bytes <= 64 * n + (int64_t(4) << 20);
}

static int64_t grid_blocks(int64_t n) { return (n + 255) / 256; }

template <typename K>
static int build_map_impl(const int32_t *coords, submconv_rulebook *rb, hipStream_t stream)
{
    const int64_t n = rb->n;
    const int path = n <= SMALL_N ? (rb->nbits <= SMALL_BITS ? 0 : 1) : (use_bitmap(n, rb->nbits) ? 2 : 3);
    auto up = [](size_t b) { return (b + 255) & ~size_t(255); };
    const int64_t words = rb->nbits > 6 ? (int64_t(1) << (rb->nbits - 6)) : 1;  // 64-bit bitmap words
    size_t off = 0, o_keys = 0, o_vals = 0, o_bm = 0, o_pre = 0, o_aux = 0;
    const size_t o_cnt = off;  // present count per block of 256 voxels
    off += up((size_t)grid_blocks(n) * 4);
    if (path == 2) {
        o_keys = off; off += up((size_t)n * sizeof(K));
        o_bm = off; off += up((size_t)(words + 1) * 8);  // +1: a 3-cell window may touch the next word
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
    uint32_t *blk_taps = (uint32_t *)(scratch + o_cnt);
    int status = SUBMCONV_OK;
    bool synced = false;  // the status read has synchronised the stream
    const unsigned grid = (unsigned)((n + 255) / 256);
    do {
        // one launch clears the status block and (dense path) the bitmap
        const int64_t clear_words = path == 2 ? words + 1 : 0;
        hipLaunchKernelGGL(k_clear, dim3((unsigned)(clear_words > 0 ? (clear_words + 4095) / 4096 : 1)), dim3(256), 0,
                           stream, st, (unsigned long long *)(scratch + o_bm), clear_words);
        if (path == 0 || path == 1) {
            if (path == 0)
                hipLaunchKernelGGL(k_build_small_bm<K>, dim3(1), dim3(1024), 0, stream, (const int4 *)coords,
                                   (int)n, rb->res, rb->batch, rb->rb, rb->nbits, (K *)rb->keys, rb->perm, rb->nbr_sp, st);
            else
                hipLaunchKernelGGL(k_build_small<K>, dim3(1), dim3(1024), 0, stream, (const int4 *)coords,
                                   (int)n, rb->res, rb->batch, rb->rb, (K *)rb->keys, rb->perm, rb->nbr_sp, st);
            hipLaunchKernelGGL(k_group_windows, dim3(grid), dim3(256), 0, stream, rb->nbr_sp, n, rb->gwin);
        } else if (path == 2) {
            K *tmp = (K *)(scratch + o_keys);
            unsigned long long *bm = (unsigned long long *)(scratch + o_bm);
            uint32_t *pre = (uint32_t *)(scratch + o_pre);
            hipLaunchKernelGGL(k_mark<K>, dim3((unsigned)((n + 256 * MARK_ROWS - 1) / (256 * MARK_ROWS))), dim3(256),
                               0, stream, (const int4 *)coords, n, rb->res, rb->batch, rb->rb, tmp, bm, st);
            // the total number of set bits lands in st->count: below n means a duplicate.  The
            // scan leaves per-tile prefixes; rank and resolve add the tile offsets (tsum).
            if ((status = exclusive_scan_u32((const uint32_t *)bm, pre, words, (uint32_t *)&st->count,
                                             scratch + o_aux, stream, SCAN_POPC64, false)) != SUBMCONV_OK) break;
            const uint32_t *tsum = (const uint32_t *)(scratch + o_aux);
            hipLaunchKernelGGL(k_rank<K>, dim3(grid), dim3(256), 0, stream, (const K *)tmp, n, bm, pre, tsum,
                               (K *)rb->keys, rb->perm);
            hipLaunchKernelGGL(k_resolve_bm<K>, dim3(grid), dim3(256), 0, stream, (const K *)rb->keys, n,
                               rb->res, rb->rb, rb->batch, bm, pre, tsum, rb->nbr_sp, rb->gwin, blk_taps);
        } else {
            K *keys_b = (K *)(scratch + o_keys);
            int32_t *vals_b = (int32_t *)(scratch + o_vals);
            const bool in_b = radix_sort_passes(n, rb->nbits) & 1;  // lands in rb->keys without a copy
            hipLaunchKernelGGL(k_pack<K>, dim3(grid), dim3(256), 0, stream, (const int4 *)coords, n,
                               rb->res, rb->batch, rb->rb, in_b ? keys_b : (K *)rb->keys,
                               in_b ? vals_b : rb->perm, st);
            if ((status = radix_sort_pairs<K>((K *)rb->keys, rb->perm, keys_b, vals_b, n, rb->nbits,
                                              scratch + o_aux, stream, in_b)) != SUBMCONV_OK) break;
            hipLaunchKernelGGL(k_resolve_win<K>, dim3(grid), dim3(256), 0, stream, (const K *)rb->keys, n,
                               rb->res, rb->rb, rb->nbr_sp, rb->gwin, blk_taps, st);
        }
        if (hipGetLastError() != hipSuccess) { status = fail(SUBMCONV_E_HIP, "kernel launch in build_map failed"); break; }
        // The staging plan is queued before the status read so it runs under the host
        // round trip; it also sums the per-block tap counts of the large-set paths.
        if ((status = win_plan_build(rb, path >= 2 ? blk_taps : nullptr, (int64_t)grid, st, stream)) != SUBMCONV_OK) break;
        DevStatus h;
        if ((status = read_status(st, &h, stream)) != SUBMCONV_OK) break;
        synced = true;
        if (path == 2 && !(h.flags & FLAG_RANGE) && (int64_t)(uint32_t)h.count != n) h.flags |= FLAG_DUPLICATE;
        if (h.flags & FLAG_RANGE) status = fail(SUBMCONV_E_COORD_RANGE, "a coordinate is outside [0,res) or its batch index outside [0,batch)");
        else if (h.flags & FLAG_DUPLICATE) status = fail(SUBMCONV_E_DUPLICATE, "the coordinate set holds a duplicate row");
        rb->taps = (int64_t)h.taps;
    } while (0);
    if (synced) dev_free_idle(scratch, stream);
    else dev_free(scratch, stream);
    return status;
}

int build_map(const int32_t *coords, submconv_rulebook *rb, hipStream_t stream)
{
    return rb->key_bytes == 4 ? build_map_impl<uint32_t>(coords, rb, stream)
                              : build_map_impl<uint64_t>(coords, rb, stream);
}

}  // namespace sc
