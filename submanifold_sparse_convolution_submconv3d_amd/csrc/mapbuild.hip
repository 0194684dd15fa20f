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
//   perm[s]       the input row of sorted voxel s,
//   nbr_sp[s]     the SORTED POSITIONS of the voxels at key[s] + offset(k), in the
//                 row form of NBR_INTS ints (common.h): per (dz, dy) row the first
//                 present position and presence bits, 40 bytes instead of 108,
//   plan[t]       per tile of 128 sorted voxels, the staging plan of the windowed
//                 forward kernel (winplan.h), built from the group windows: per
//                 group of 32 consecutive sorted voxels and per (dz, dy) row, the
//                 first and last sorted position the group's neighbours in that row
//                 occupy (kept in LDS, or in gwin[] by the sparse path),
//   keys[s]       the sorted keys.
// The input-order table nbr[i][k] (input rows) is derived from these on request.
//
// Dense key space (2^nbits bitmap bits affordable next to N), six launches:
//   clear    - zero the status block, the occupancy bitmap and the scan's flags;
//   mark     - validate and pack each row's key and set its bit in the bitmap
//              (a per-block LDS hash of bitmap words first, then one device-scope
//              OR per distinct word and block);
//   scan     - single-pass exclusive scan of the words' popcounts (decoupled
//              look-back across blocks): every word's global prefix and the
//              distinct-key count (a count below N means a duplicate);
//   rank     - input row i with key k sits at sorted position prefix[k / 64] + (set
//              bits of its word below k): one radix pass whose digit is the whole key;
//   resolve + plan - each block of 256 sorted positions forms each neighbour row
//              from three bits and one rank query per (dz, dy) row, writes the rows as
//              coalesced runs, and computes the staging plans of its two tiles from
//              its waves' row windows in LDS;
//   post     - one block sums the resolve blocks' present counts and writes the
//              status to the host's pinned mailbox, which the call polls (no copy and
//              no stream synchronisation).
// Sparse key space (huge grid, few voxels):
//   pack + multi-pass LSD radix sort, then per tile of 256 sorted voxels: the x
//   neighbours of the centre row are the adjacent sorted entries; for each of the
//   other 8 (dz, dy) rows every target key lies in [first + off - 1, last + off + 1]
//   (off = the row's key offset), so the block copies that window of sorted keys
//   into LDS and binary-searches there (a window too big for LDS is searched in
//   place).
// Small sets (n <= 2048) build in one block, which also posts the status to the
// host's mailbox itself (one launch in all).  Coordinates are range-checked
// before packing and every neighbour coordinate is bounds-checked before its key
// is formed, so a key never wraps into the next row, plane or batch entry.
#include "common.h"
#include "mailbox.h"
#include "winplan.h"

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
constexpr uint32_t MARK_EMPTY = ~0u;  // word indices are below 2^25 (keys of at most 31 bits)

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
    __shared__ __attribute__((aligned(16))) uint32_t s_word[MARK_SLOTS];
    __shared__ __attribute__((aligned(16))) unsigned long long s_bits[MARK_SLOTS];
    for (int i = threadIdx.x; i < MARK_SLOTS / 4; i += 256)
        ((uint4 *)s_word)[i] = make_uint4(MARK_EMPTY, MARK_EMPTY, MARK_EMPTY, MARK_EMPTY);
    for (int i = threadIdx.x; i < MARK_SLOTS / 2; i += 256) ((ulonglong2 *)s_bits)[i] = make_ulonglong2(0ull, 0ull);
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
            const uint32_t w = (uint32_t)(key >> 6);
            uint32_t h = (w * 0x9E3779B1u) >> (32 - 11);
            // linear probing; the table has twice the block's rows, so it never fills
            for (;;) {
                const uint32_t prev = atomicCAS(&s_word[h], MARK_EMPTY, w);
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
        const uint32_t w = s_word[i];
        if (w != MARK_EMPTY) atomicOr(&bm[w], s_bits[i]);
    }
}

// Single-pass exclusive scan of the bitmap words' popcounts.  Tile t (one block)
// covers `chunks` runs of 256 x WPT words.  Its total is published in look[t] at once
// (flag LB_AGG); wave 0 then walks back over its predecessors 64 at a time, adding
// aggregates until it meets an inclusive prefix (flag LB_INCL; the space before tile
// 0 counts as an inclusive 0), and publishes its own inclusive prefix.  Every block
// waits only on lower-numbered blocks, and the grid is kept small enough
// (SK_MAX_TILES) to be resident at once, so every wait ends.  Every word then gets its
// global exclusive prefix.  The grand total goes to st->count (below n means a
// duplicate or an invalid row).
constexpr int SK_MAX_TILES = 1024;
constexpr unsigned long long LB_AGG = 1ull << 62, LB_INCL = 1ull << 63, LB_VAL = 0xffffffffull;

template <int WPT>
__device__ __forceinline__ void sk_words(const unsigned long long *__restrict__ bm, int64_t words, int64_t w0,
                                         unsigned long long (&v)[WPT])
{
    if (w0 + WPT <= words) {
        const ulonglong2 *src = (const ulonglong2 *)(bm + w0);  // w0 is a multiple of WPT (even)
#pragma unroll
        for (int h = 0; h < WPT / 2; ++h) {
            const ulonglong2 x = src[h];
            v[2 * h] = x.x;
            v[2 * h + 1] = x.y;
        }
    } else {
#pragma unroll
        for (int e = 0; e < WPT; ++e) v[e] = w0 + e < words ? bm[w0 + e] : 0ull;
    }
}

template <int WPT>
__global__ __launch_bounds__(256) void k_scan_words(const unsigned long long *__restrict__ bm, int64_t words,
                                                    int chunks, uint32_t *__restrict__ prefix,
                                                    unsigned long long *look, DevStatus *st)
{
    constexpr int CH = 256 * WPT;  // words per chunk
    __shared__ uint32_t s_red[4];
    __shared__ uint32_t s_excl;
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t t = blockIdx.x;
    const int64_t base = t * (int64_t)chunks * CH;
    uint32_t local = 0;
    for (int c = 0; c < chunks; ++c) {
        unsigned long long v[WPT];
        sk_words<WPT>(bm, words, base + (int64_t)c * CH + tid * WPT, v);
#pragma unroll
        for (int e = 0; e < WPT; ++e) local += (uint32_t)__popcll(v[e]);
    }
    uint32_t tile_total;
    const uint32_t incl = block_incl_scan256(local, s_red, &tile_total);
    if (tid == 0)
        __hip_atomic_store(look + t, (t == 0 ? LB_INCL : LB_AGG) | tile_total, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    if (tid < 64) {
        uint32_t excl = 0;
        int64_t j = t - 1;  // newest predecessor not yet added
        while (j >= 0) {
            const int64_t idx = j - lane;
            unsigned long long v = LB_INCL;  // before tile 0: an inclusive prefix of 0
            if (idx >= 0) {
                v = __hip_atomic_load(look + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                while (!(v & (LB_AGG | LB_INCL))) {
                    __builtin_amdgcn_s_sleep(1);
                    v = __hip_atomic_load(look + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            const uint64_t inc = __ballot((v & LB_INCL) != 0);
            const int stop = inc ? __ffsll((unsigned long long)inc) - 1 : 63;  // first inclusive lane
            uint32_t add = lane <= stop ? (uint32_t)(v & LB_VAL) : 0u;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) add += __shfl_xor(add, off, 64);
            excl += add;
            if (inc) break;
            j -= 64;
        }
        if (lane == 0) {
            if (t > 0)
                __hip_atomic_store(look + t, LB_INCL | (excl + tile_total), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            s_excl = excl;
            if (t == (int64_t)gridDim.x - 1) st->count = (unsigned long long)(excl + tile_total);
        }
    }
    __syncthreads();
    uint32_t run = s_excl + incl - local;
    for (int c = 0; c < chunks; ++c) {
        const int64_t cw0 = base + (int64_t)c * CH;
        const int64_t w0 = cw0 + tid * WPT;
        unsigned long long v[WPT];
        sk_words<WPT>(bm, words, w0, v);
        uint32_t pre[WPT];
#pragma unroll
        for (int e = 0; e < WPT; ++e) {
            pre[e] = run;
            run += (uint32_t)__popcll(v[e]);
        }
        if (w0 + WPT <= words) {
            if constexpr (WPT % 4 == 0) {
                uint4 *dst = (uint4 *)(prefix + w0);
#pragma unroll
                for (int h = 0; h < WPT / 4; ++h) dst[h] = make_uint4(pre[4 * h], pre[4 * h + 1], pre[4 * h + 2], pre[4 * h + 3]);
            } else {
#pragma unroll
                for (int e = 0; e < WPT; ++e) prefix[w0 + e] = pre[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < WPT; ++e)
                if (w0 + e < words) prefix[w0 + e] = pre[e];
        }
    }
}

// Rank: input row i with key k sits at sorted position prefix[k / 64] + (set bits of
// its word below k), one radix pass whose digit is the whole key: perm[s] = i and
// sk[s] = k.
template <typename K>
__global__ __launch_bounds__(256) void k_rank(const K *__restrict__ keys_in, int64_t n,
                                              const unsigned long long *__restrict__ bm,
                                              const uint32_t *__restrict__ prefix, K *__restrict__ sk,
                                              int32_t *__restrict__ perm)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const K key = keys_in[i];
    if (key == (K)~K(0)) return;  // an invalid row (reported by the build) has no position
    const uint64_t w = (uint64_t)(key >> 6);
    const uint32_t r = prefix[w] + (uint32_t)__popcll(bm[w] & ((1ull << (uint32_t)(key & 63)) - 1ull));
    if (r < (uint64_t)n) {
        sk[r] = key;
        perm[r] = (int32_t)i;
    }
}

// Resolve and staging plan: each block resolves RR_T sorted positions (two plan
// tiles).  For each (dz, dy) row d the voxel's neighbours at x - 1, x, x + 1 are three
// consecutive bits of the occupancy bitmap, read as one funnel shift of two 32-bit
// halves, and the first of them has the rank prefix + (set bits before it); the
// present cells of a row take consecutive positions from there.  The rows are written
// as coalesced runs through LDS; the row windows of each wave (per 64 voxels and row d:
// first and last position of the neighbours) stay in LDS and give the plans of the
// block's two tiles (plan_tile_team).  The block's present count goes to blk_taps
// (summed by k_post_status).  Positions at or past st->count (the distinct keys; fewer
// than n only for an invalid set, which the build reports) are not resolved.
constexpr int RR_T = 256;  // sorted voxels per resolve block
static_assert(RR_T == 2 * WIN_TILE, "a resolve block plans two tiles");

template <typename K, bool WORDROWS>
__global__ __launch_bounds__(256) void k_resolve_plan(const K *__restrict__ sk, int64_t n, int res, int rb,
                                                      const unsigned long long *__restrict__ bm, int bm_bytes,
                                                      const uint32_t *__restrict__ prefix, int pre_bytes,
                                                      int32_t *__restrict__ nbr_sp, int32_t *__restrict__ plan,
                                                      int64_t ntiles, const DevStatus *st,
                                                      uint32_t *__restrict__ blk_taps)
{
    __shared__ __attribute__((aligned(16))) int32_t s_rows[RR_T * NBR_INTS];
    __shared__ int32_t s_win[4 * 18];
    __shared__ __attribute__((aligned(16))) int32_t s_rec[2 * PLAN_INTS];
    __shared__ uint32_t s_wt[4];
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t blk = blockIdx.x;
    const int64_t s0 = blk * RR_T;
    const int count = (int)((n - s0) < RR_T ? (n - s0) : RR_T);
    const int64_t limit = (int64_t)st->count < n ? (int64_t)st->count : n;
    const int64_t s = s0 + tid;
    const bool valid = s < limit;
    const K key = valid ? sk[s] : K(0);
    const K m = (K(1) << rb) - 1;
    const int x = (int)(key & m), y = (int)((key >> rb) & m), z = (int)((key >> (2 * rb)) & m);
    const bool xlo = x > 0, xhi = x + 1 < res;
    const K base = key - (xlo ? K(1) : K(0));  // each row's window starts at cell x - 1 (x when x = 0)
    const uint32_t shift = xlo ? 0u : 1u;      // window bit j <-> cell x - 1 + j
    const uint32_t valid3 = (xlo ? 1u : 0u) | 2u | (xhi ? 4u : 0u);
    const bool zok[3] = {z > 0, true, z + 1 < res}, yok[3] = {y > 0, true, y + 1 < res};
    int32_t r[NBR_INTS];
    uint32_t mask = 0;
    if constexpr (WORDROWS) {
        // At least 6 bits per axis: every (dz, dy) row offset is a whole number of 64-bit
        // words, so the nine windows share their bit position in the word, and their words
        // are the centre word plus per-row constants.  Words and prefixes are read through
        // bounds-checked buffers (a row off the grid may form an offset outside them, which
        // reads zeros; its bits are masked either way).
        const __amdgpu_buffer_rsrc_t rbm = __builtin_amdgcn_make_buffer_rsrc((void *)bm, (short)0, bm_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rpre = __builtin_amdgcn_make_buffer_rsrc((void *)prefix, (short)0, pre_bytes, 0x00020000);
        const uint32_t wb = (uint32_t)((uint64_t)base >> 6), b = (uint32_t)(base & 63);
        const bool up = b >= 32;
        const uint32_t sh = b & 31u, m = (1u << sh) - 1u;
        const uint32_t mlo = up ? ~0u : m, mhi = up ? m : 0u;  // bits of the word before the window
        const int32_t row_w = 1 << (rb - 6), plane_w = 1 << (2 * rb - 6);
        uint32_t lo[9], hi[9], nx[9], pre[9];
#pragma unroll
        for (int d = 0; d < 9; ++d) {
            const int dz = d / 3 - 1, dy = d % 3 - 1;
            const uint32_t w = wb + (uint32_t)(dz * plane_w + dy * row_w);
            // the word and the low half of the next one (the bitmap has one word of padding)
            const auto v = __builtin_amdgcn_raw_buffer_load_b96(rbm, w * 8u, 0, 0);
            lo[d] = v[0];
            hi[d] = v[1];
            nx[d] = v[2];
            pre[d] = d == 4 ? 0u : __builtin_amdgcn_raw_buffer_load_b32(rpre, w * 4u, 0, 0);
        }
#pragma unroll
        for (int d = 0; d < 9; ++d) {
            const int dz = d / 3 - 1, dy = d % 3 - 1;
            // cells of the row on the grid (none for a row off it): a mask, not a branch
            const uint32_t vm = (valid && zok[dz + 1] && yok[dy + 1]) ? valid3 : 0u;
            const uint32_t cur = up ? hi[d] : lo[d], nxt = up ? nx[d] : hi[d];
            const uint32_t bits = (__builtin_amdgcn_alignbit(nxt, cur, sh) << shift) & vm;
            // the centre row's window starts at the voxel itself or the one before it
            r[d] = d == 4 ? (int32_t)((uint32_t)s - (bits & 1u))
                          : (int32_t)(pre[d] + (uint32_t)__popc(lo[d] & mlo) + (uint32_t)__popc(hi[d] & mhi));
            mask |= bits << (3 * d);
        }
    } else {
        const uint32_t *bm32 = (const uint32_t *)bm;
        // every load first (rows off the grid read word 0 and are masked): one round trip
        unsigned long long wv[9];
        uint32_t nx[9], pre[9], bsh[9];
        bool rok[9];
#pragma unroll
        for (int d = 0; d < 9; ++d) {
            const int dz = d / 3 - 1, dy = d % 3 - 1;
            rok[d] = valid && zok[dz + 1] && yok[dy + 1];
            const K off = (K)((int64_t)dz << (2 * rb)) + (K)((int64_t)dy << rb);  // wraps correctly for dz, dy < 0
            const K c0 = rok[d] ? (K)(base + off) : K(0);
            const uint64_t w = (uint64_t)(c0 >> 6);
            bsh[d] = (uint32_t)(c0 & 63);
            wv[d] = bm[w];
            nx[d] = bm32[2 * w + 2];  // low half of the next word (the bitmap has one word of padding)
            pre[d] = d == 4 ? 0u : prefix[w];
        }
#pragma unroll
        for (int d = 0; d < 9; ++d) {
            const uint32_t b = bsh[d], lo32 = (uint32_t)wv[d], hi32 = (uint32_t)(wv[d] >> 32);
            const bool up = b >= 32;
            const uint32_t cur = up ? hi32 : lo32, nxt = up ? nx[d] : hi32, below = up ? lo32 : 0u;
            const uint32_t sh = b & 31u;
            uint32_t bits = __builtin_amdgcn_alignbit(nxt, cur, sh) & 7u;
            bits = rok[d] ? ((bits << shift) & valid3) : 0u;
            r[d] = d == 4 ? (int32_t)((uint32_t)s - (bits & 1u))
                          : (int32_t)(pre[d] + (uint32_t)__popc(below) + (uint32_t)__popc(cur & ((1u << sh) - 1u)));
            mask |= bits << (3 * d);
        }
    }
    r[9] = (int32_t)mask;
    if (tid < count) {
#pragma unroll
        for (int q = 0; q < NBR_INTS; ++q) s_rows[tid * NBR_INTS + q] = r[q];
    }
    // The window of each (dz, dy) row over the wave's 64 voxels: the row's first position
    // in the first lane that has the row, its last in the last such lane (windows are
    // monotone in sorted order, see group_windows_write).  Found with one ballot and
    // scalar lane lookups per row; lane 0 stores the wave's 9 starts, then its 9 ends.
    {
        int32_t wlo[9], whi[9];
#pragma unroll
        for (int d = 0; d < 9; ++d) {
            const uint32_t bits = (mask >> (3 * d)) & 7u;
            const uint64_t bal = __ballot(bits != 0u);
            wlo[d] = GWIN_NONE;
            whi[d] = -1;
            if (bal) {
                const int f = __builtin_ctzll(bal), l = 63 - __builtin_clzll(bal);
                wlo[d] = __builtin_amdgcn_readlane(r[d], f);
                whi[d] = __builtin_amdgcn_readlane(r[d], l) +
                         __popc((uint32_t)__builtin_amdgcn_readlane((int)bits, l)) - 1;
            }
        }
        if (lane == 0) {
#pragma unroll
            for (int d = 0; d < 9; ++d) {
                s_win[(tid >> 6) * 18 + d] = wlo[d];
                s_win[(tid >> 6) * 18 + 9 + d] = whi[d];
            }
        }
    }
    uint32_t present = (uint32_t)__popc(mask);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) present += __shfl_xor(present, off, 64);
    if (lane == 0) s_wt[tid >> 6] = present;
    __syncthreads();
    // rows out as one contiguous run (the block's rows start 16-byte aligned)
    {
        const int ints = count * NBR_INTS, v4 = ints >> 2;
        int4 *dst = (int4 *)(nbr_sp + s0 * NBR_INTS);
        const int4 *src = (const int4 *)s_rows;
        for (int e = tid; e < v4; e += 256) dst[e] = src[e];
        for (int e = 4 * v4 + tid; e < ints; e += 256) nbr_sp[s0 * NBR_INTS + e] = s_rows[e];
    }
    // the two tiles' staging plans (wave 0: a team of 16 lanes per tile, the tile's two
    // waves' windows joined; an empty window is (GWIN_NONE, -1))
    if (tid < 64) {
        const int team = (tid >> 4) & 1, q = tid & 15;
        int32_t lo = GWIN_NONE, hi = -1;
        if (q < 9) {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                lo = min(lo, s_win[(2 * team + g) * 18 + q]);
                hi = max(hi, s_win[(2 * team + g) * 18 + 9 + q]);
            }
        }
        if (tid < 32) plan_tile_team(lo, hi, q, WIN_CAP, s_rec + team * PLAN_INTS);
    }
    __syncthreads();
    if (tid < 2 * PLAN_INTS) {
        const int64_t tile = 2 * blk + (tid >> 5);
        if (tile < ntiles) plan[tile * PLAN_INTS + (tid & 31)] = s_rec[tid];
    }
    if (tid == 0) blk_taps[blk] = s_wt[0] + s_wt[1] + s_wt[2] + s_wt[3];
}

// The build's status and the sum of the resolve blocks' present counts, posted to the
// host's mailbox by one block after the resolve has ended (so every write of the build
// is visible device-wide when the host sees the post).  Counting the blocks inside the
// resolve instead cost more: a device-scope fence per block writes back the XCD's L2,
// and a returning device atomic per block holds each block for a round trip to memory.
__global__ __launch_bounds__(1024) void k_post_status(const DevStatus *st, const uint32_t *__restrict__ blk_taps,
                                                      int64_t nblk, Mailbox *mb, uint32_t seq)
{
    __shared__ unsigned long long s_part[16];
    // eight independent loads per step, so a step costs one round trip to memory
    unsigned long long t = 0;
    for (int64_t i0 = threadIdx.x; i0 < nblk; i0 += 8 * 1024) {
        uint32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = i0 + u * 1024 < nblk ? blk_taps[i0 + u * 1024] : 0u;
#pragma unroll
        for (int u = 0; u < 8; ++u) t += v[u];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off, 64);
    if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = t;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long taps = st->taps;
        for (int w = 0; w < 16; ++w) taps += s_part[w];
        mailbox_post(mb, seq, st->flags, taps, st->count);
    }
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

// End of a single-block build (every thread calls it, rows of all n sorted voxels in
// s_rows): the rows go out as one run, the group windows are formed per 32 sorted
// voxels in LDS, each tile's staging plan is computed by a team of 16 lanes, and the
// status goes to the host's mailbox once every wave's stores have completed (they all
// sit in this CU's L2, which the posting thread's system-scope release writes back),
// so the call needs no copy and no stream synchronisation.
__device__ void small_finish(const int32_t *s_rows, int n, int32_t *__restrict__ nbr_sp,
                             int32_t *__restrict__ plan, int32_t *s_gwin, int32_t *s_rec, uint32_t flags,
                             uint32_t taps, Mailbox *mb, uint32_t seq)
{
    const int tid = threadIdx.x;
    for (int e = tid; e < n * NBR_INTS; e += 1024) nbr_sp[e] = s_rows[e];
    const int ngroups = (n + 31) >> 5;
    for (int h = 0; h < SMALL_N / 1024; ++h) {
        const int s = tid + 1024 * h;
        int32_t r[NBR_INTS];
#pragma unroll
        for (int q = 0; q < NBR_INTS; ++q) r[q] = s < n ? s_rows[s * NBR_INTS + q] : 0;
        group_windows_write_row(r, s < n, s >> 5, ngroups, s_gwin);
    }
    __syncthreads();
    const int ntiles = (n + WIN_TILE - 1) / WIN_TILE, team = tid >> 4, q = tid & 15;
    int32_t lo = GWIN_NONE, hi = -1;
    if (team < ntiles && q < 9) {
        for (int g = 4 * team; g < 4 * team + 4 && g < ngroups; ++g) {
            const int32_t wl = s_gwin[g * GWIN_INTS + q], wh = s_gwin[g * GWIN_INTS + 9 + q];
            if (wh >= 0) {
                lo = min(lo, wl);
                hi = max(hi, wh);
            }
        }
    }
    if (team < SMALL_N / WIN_TILE) plan_tile_team(lo, hi, q, WIN_CAP, s_rec + team * PLAN_INTS);
    __syncthreads();
    for (int e = tid; e < ntiles * PLAN_INTS; e += 1024) plan[e] = s_rec[e];
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
    __syncthreads();
    if (tid == 0) mailbox_post(mb, seq, flags, taps, (unsigned long long)n);
}

// Key space of at most 2^16 bits: bitmap and prefix in LDS.
template <typename K>
__global__ __launch_bounds__(1024) void k_build_small_bm(const int4 *__restrict__ coords, int n,
                                                         int res, int batch, int rb, int nbits,
                                                         K *__restrict__ keys_out,
                                                         int32_t *__restrict__ perm_out,
                                                         int32_t *__restrict__ nbr_sp, int32_t *__restrict__ plan,
                                                         Mailbox *mb, uint32_t seq)
{
    constexpr int WORDS = (1 << SMALL_BITS) / 32;
    __shared__ uint32_t s_bm[WORDS];
    __shared__ uint32_t s_pre[WORDS];
    __shared__ uint32_t s_wave[16];
    __shared__ uint32_t s_flags, s_taps;
    __shared__ int32_t s_rows[SMALL_N * NBR_INTS];
    __shared__ int32_t s_gwin[SMALL_N / 32 * GWIN_INTS];
    __shared__ int32_t s_rec[SMALL_N / 16 * PLAN_INTS];
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
        uint32_t before = 0;  // the totals of the waves before this one (16 reads issued together)
#pragma unroll
        for (int w = 0; w < 16; ++w) before += w < (int)wave ? s_wave[w] : 0u;
        const uint32_t ex = x - v + before;
        if (w0 < words) s_pre[w0] = ex;
        if (w0 + 1 < words) s_pre[w0 + 1] = ex + a;
    }
    __syncthreads();
    if (s_flags) {  // invalid set: report only (nothing was written)
        if (tid == 0) mailbox_post(mb, seq, s_flags, 0ull, 0ull);
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
        // the 27 lookups without branches: every word and prefix is read (at key 0 for a
        // neighbour off the grid, which is then masked), all reads issued together
        int32_t p[27];
        uint32_t word[27], pre[27], bit[27];
        bool on[27];
#pragma unroll
        for (int k = 0; k < 27; ++k) {
            const int nz = z + k / 9 - 1, ny = y + (k / 3) % 3 - 1, nx = x + k % 3 - 1;
            on[k] = nz >= 0 && nz < res && ny >= 0 && ny < res && nx >= 0 && nx < res;
            const K t = on[k] ? (bpart | ((K)nz << (2 * rb)) | ((K)ny << rb) | (K)nx) : K(0);
            bit[k] = (uint32_t)(t & 31);
            word[k] = s_bm[t >> 5];
            pre[k] = s_pre[t >> 5];
        }
#pragma unroll
        for (int k = 0; k < 27; ++k) {
            const bool hit = on[k] && ((word[k] >> bit[k]) & 1u);
            const int32_t r = hit ? (int32_t)(pre[k] + __popc(word[k] & ((1u << bit[k]) - 1u))) : -1;
            present += r >= 0;
            p[k] = r;
        }
        int32_t rr[NBR_INTS];
        nbr_pack(p, rr);
#pragma unroll
        for (int q = 0; q < NBR_INTS; ++q) s_rows[s * NBR_INTS + q] = rr[q];
    }
    if (present) atomicAdd(&s_taps, present);
    __syncthreads();
    small_finish(s_rows, n, nbr_sp, plan, s_gwin, s_rec, 0u, s_taps, mb, seq);
}

// Larger key space: bitonic sort of (key, row) in LDS, binary search in LDS.
template <typename K>
__global__ __launch_bounds__(1024) void k_build_small(const int4 *__restrict__ coords, int n,
                                                      int res, int batch, int rb,
                                                      K *__restrict__ keys_out,
                                                      int32_t *__restrict__ perm_out,
                                                      int32_t *__restrict__ nbr_sp, int32_t *__restrict__ plan,
                                                      Mailbox *mb, uint32_t seq)
{
    __shared__ K s_key[SMALL_N];
    __shared__ int32_t s_row[SMALL_N];
    __shared__ uint32_t s_red[2];
    __shared__ int32_t s_rows[SMALL_N * NBR_INTS];
    __shared__ int32_t s_gwin[SMALL_N / 32 * GWIN_INTS];
    __shared__ int32_t s_rec[SMALL_N / 16 * PLAN_INTS];
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
    if (tid == 0) s_red[0] = s_red[1] = 0;
    __syncthreads();
    if (bad_any) atomicOr(&s_red[1], FLAG_RANGE);
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
        if (s + 1 < n && s_key[s + 1] == key) atomicOr(&s_red[1], FLAG_DUPLICATE);
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
        for (int q = 0; q < NBR_INTS; ++q) s_rows[s * NBR_INTS + q] = rr[q];
    }
    if (present) atomicAdd(&s_red[0], present);
    __syncthreads();
    small_finish(s_rows, n, nbr_sp, plan, s_gwin, s_rec, s_red[1], s_red[0], mb, seq);
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

// Zero the status block, `words` 64-bit words at w (the bitmap) and `words2` at w2
// (the scan's look-back flags); grid-stride.
__global__ __launch_bounds__(256) void k_clear(DevStatus *st, unsigned long long *__restrict__ w, int64_t words,
                                               unsigned long long *__restrict__ w2, int64_t words2)
{
    if (blockIdx.x == 0 && threadIdx.x == 0) *st = DevStatus{};
    // pairs of words as 16-byte stores (w is 16-byte aligned), then an odd last word
    const int64_t pairs = words >> 1;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < pairs; i += (int64_t)gridDim.x * 256)
        ((ulonglong2 *)w)[i] = make_ulonglong2(0ull, 0ull);
    if ((words & 1) && blockIdx.x == 0 && threadIdx.x == 0) w[words - 1] = 0ull;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words2; i += (int64_t)gridDim.x * 256) w2[i] = 0ull;
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
    const int64_t ntiles = (n + WIN_TILE - 1) / WIN_TILE;
    // dense path: scan tiles of `chunks` x 256 x wpt words, at most SK_MAX_TILES of them (2 words per
    // thread while that keeps enough tiles busy, else 8)
    const int wpt = words <= (int64_t)512 * SK_MAX_TILES ? 2 : 8;
    const int64_t chw = (int64_t)256 * wpt;
    const int chunks = (int)((words + chw * SK_MAX_TILES - 1) / (chw * SK_MAX_TILES));
    const int64_t stiles = (words + (int64_t)chunks * chw - 1) / ((int64_t)chunks * chw);
    const int64_t rblocks = (n + RR_T - 1) / RR_T;  // resolve blocks of the dense path
    // the status block first, then the per-block present counts (dense and sparse paths)
    size_t off = up(sizeof(DevStatus) + (size_t)(path == 2 ? rblocks : (path == 3 ? grid_blocks(n) : 0)) * 4);
    size_t o_keys = 0, o_vals = 0, o_bm = 0, o_pre = 0, o_aux = 0;
    if (path == 2) {
        o_keys = off; off += up((size_t)n * sizeof(K));
        o_bm = off; off += up((size_t)(words + 1) * 8);  // +1: a 3-cell window may touch the next word
        o_pre = off; off += up((size_t)words * 4);
        o_aux = off; off += up((size_t)stiles * 8);      // look-back flags of the scan
    } else if (path == 3) {
        o_keys = off; off += up((size_t)n * sizeof(K));
        o_vals = off; off += up((size_t)n * 4);
        o_aux = off; off += up(sort_scratch_bytes(n));
    }
    char *scratch = nullptr;  // none for the single-block builds
    if (path >= 2) SC_CHECK(dev_alloc((void **)&scratch, off, stream));
    DevStatus *st = (DevStatus *)scratch;
    uint32_t *blk_taps = scratch ? (uint32_t *)(scratch + sizeof(DevStatus)) : nullptr;
    int status = SUBMCONV_OK;
    bool synced = false;  // the status read has synchronised the stream
    Mailbox *mb = nullptr;
    uint32_t mb_seq = 0;
    const unsigned grid = (unsigned)((n + 255) / 256);
    do {
        // one launch clears the status block and (dense path) the bitmap and the scan's flags;
        // the single-block builds need no clearing (they post their status themselves)
        const int64_t clear_words = path == 2 ? words + 1 : 0;
        if (path >= 2)
            hipLaunchKernelGGL(k_clear, dim3((unsigned)(clear_words > 0 ? (clear_words + 4095) / 4096 : 1)), dim3(256),
                               0, stream, st, (unsigned long long *)(scratch + o_bm), clear_words,
                               (unsigned long long *)(scratch + o_aux), path == 2 ? stiles : int64_t(0));
        if (path == 0 || path == 1) {
            if ((status = mailbox_acquire(&mb, &mb_seq)) != SUBMCONV_OK) break;
            if (path == 0)
                hipLaunchKernelGGL(k_build_small_bm<K>, dim3(1), dim3(1024), 0, stream, (const int4 *)coords,
                                   (int)n, rb->res, rb->batch, rb->rb, rb->nbits, (K *)rb->keys, rb->perm, rb->nbr_sp,
                                   rb->plan, mb, mb_seq);
            else
                hipLaunchKernelGGL(k_build_small<K>, dim3(1), dim3(1024), 0, stream, (const int4 *)coords,
                                   (int)n, rb->res, rb->batch, rb->rb, (K *)rb->keys, rb->perm, rb->nbr_sp, rb->plan,
                                   mb, mb_seq);
        } else if (path == 2) {
            K *tmp = (K *)(scratch + o_keys);
            unsigned long long *bm = (unsigned long long *)(scratch + o_bm);
            uint32_t *pre = (uint32_t *)(scratch + o_pre);
            hipLaunchKernelGGL(k_mark<K>, dim3((unsigned)((n + 256 * MARK_ROWS - 1) / (256 * MARK_ROWS))), dim3(256),
                               0, stream, (const int4 *)coords, n, rb->res, rb->batch, rb->rb, tmp, bm, st);
            // global prefixes of the words and the distinct count in st->count
            if (wpt == 2)
                hipLaunchKernelGGL(k_scan_words<2>, dim3((unsigned)stiles), dim3(256), 0, stream,
                                   (const unsigned long long *)bm, words, chunks, pre,
                                   (unsigned long long *)(scratch + o_aux), st);
            else
                hipLaunchKernelGGL(k_scan_words<8>, dim3((unsigned)stiles), dim3(256), 0, stream,
                                   (const unsigned long long *)bm, words, chunks, pre,
                                   (unsigned long long *)(scratch + o_aux), st);
            hipLaunchKernelGGL(k_rank<K>, dim3(grid), dim3(256), 0, stream, (const K *)tmp, n,
                               (const unsigned long long *)bm, (const uint32_t *)pre, (K *)rb->keys, rb->perm);
            // the bitmap (words + 1 of padding) and the prefixes are below 2^28 bytes (nbits <= 31)
            const int bm_bytes = (int)((words + 1) * 8), pre_bytes = (int)(words * 4);
            if ((status = mailbox_acquire(&mb, &mb_seq)) != SUBMCONV_OK) break;
            if (rb->rb >= 6)
                hipLaunchKernelGGL((k_resolve_plan<K, true>), dim3((unsigned)rblocks), dim3(256), 0, stream,
                                   (const K *)rb->keys, n, rb->res, rb->rb, (const unsigned long long *)bm, bm_bytes,
                                   (const uint32_t *)pre, pre_bytes, rb->nbr_sp, rb->plan, ntiles,
                                   (const DevStatus *)st, blk_taps);
            else
                hipLaunchKernelGGL((k_resolve_plan<K, false>), dim3((unsigned)rblocks), dim3(256), 0, stream,
                                   (const K *)rb->keys, n, rb->res, rb->rb, (const unsigned long long *)bm, bm_bytes,
                                   (const uint32_t *)pre, pre_bytes, rb->nbr_sp, rb->plan, ntiles,
                                   (const DevStatus *)st, blk_taps);
            hipLaunchKernelGGL(k_post_status, dim3(1), dim3(1024), 0, stream, (const DevStatus *)st,
                               (const uint32_t *)blk_taps, rblocks, mb, mb_seq);
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
        // The other paths plan from the group windows; the plan kernel also sums the sparse
        // path's per-block present counts.
        if (path == 3 && (status = win_plan_build(rb, blk_taps, (int64_t)grid, st, stream)) != SUBMCONV_OK) break;
        DevStatus h;
        uint64_t taps = 0;
        if (path <= 2) {
            // the last kernel posts the status to the mailbox: no copy, no stream synchronisation
            if ((status = mailbox_wait(mb, mb_seq, &h, stream)) != SUBMCONV_OK) break;
        } else {
            if ((status = read_status_counts(st, 0, &h, &taps, stream)) != SUBMCONV_OK) break;
            synced = true;
        }
        if (path == 2 && !(h.flags & FLAG_RANGE) && (int64_t)h.count != n) h.flags |= FLAG_DUPLICATE;
        if (h.flags & FLAG_RANGE) status = fail(SUBMCONV_E_COORD_RANGE, "a coordinate is outside [0,res) or its batch index outside [0,batch)");
        else if (h.flags & FLAG_DUPLICATE) status = fail(SUBMCONV_E_DUPLICATE, "the coordinate set holds a duplicate row");
        rb->taps = (int64_t)(h.taps + taps);
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
