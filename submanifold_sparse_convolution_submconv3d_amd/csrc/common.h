// Internal declarations of the submconv HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "submconv.h"

namespace sc {

// --------------------------------------------------------------------------
// errors
// --------------------------------------------------------------------------

// Record a printf-style detail message for submconv_last_error; returns `status`.
int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

#define SC_HIP(expr)                                                              \
    do {                                                                          \
        hipError_t e_ = (expr);                                                   \
        if (e_ != hipSuccess)                                                     \
            return ::sc::fail(e_ == hipErrorOutOfMemory ? SUBMCONV_E_OOM          \
                                                        : SUBMCONV_E_HIP,         \
                              "%s: %s", #expr, hipGetErrorString(e_));            \
    } while (0)

#define SC_LAUNCHED(name)                                                         \
    do {                                                                          \
        hipError_t e_ = hipGetLastError();                                        \
        if (e_ != hipSuccess)                                                     \
            return ::sc::fail(SUBMCONV_E_HIP, "launch of %s: %s", name,           \
                              hipGetErrorString(e_));                             \
    } while (0)

#define SC_CHECK(expr)                                                            \
    do {                                                                          \
        int s_ = (expr);                                                          \
        if (s_ != SUBMCONV_OK) return s_;                                         \
    } while (0)

// --------------------------------------------------------------------------
// device status block (one per map build / helper call)
// --------------------------------------------------------------------------

enum : uint32_t { FLAG_RANGE = 1u, FLAG_DUPLICATE = 2u };

struct DevStatus {
    uint32_t flags;              // FLAG_* bits, or-ed by kernels
    uint32_t pad;
    unsigned long long taps;     // present entries of the neighbour table
    unsigned long long count;    // an output row count (helpers)
    unsigned long long pad2;
};

// Enqueue a copy of `d` to a pinned host block, synchronise `stream`, return it in `h`.
int read_status(const DevStatus *d, DevStatus *h, hipStream_t stream);
// The same, together with `ncounts` uint32 counters stored right after `d`; their
// sum is returned in *sum.
int read_status_counts(const DevStatus *d, int64_t ncounts, DevStatus *h, uint64_t *sum, hipStream_t stream);

// A status block in coherent pinned host memory that a kernel writes itself, so the
// host learns the result by polling `seq` instead of enqueueing a copy and
// synchronising the stream.  One per host thread.
struct Mailbox {
    uint32_t seq;                // written last, to the value the host expects
    uint32_t flags;
    unsigned long long taps;
    unsigned long long count;
};
// This thread's mailbox (device-visible) and the sequence number the next post must carry.
int mailbox_acquire(Mailbox **mb, uint32_t *seq);
// Wait until `mb` carries `seq` (polling, then a stream synchronisation as a fallback)
// and return its fields in `h`.
int mailbox_wait(Mailbox *mb, uint32_t seq, DevStatus *h, hipStream_t stream);


// --------------------------------------------------------------------------
// stream-ordered device memory
// --------------------------------------------------------------------------

int dev_alloc(void **p, size_t bytes, hipStream_t stream);
void dev_free(void *p, hipStream_t stream);
// dev_free for a block whose stream has just been synchronised (no pending use)
void dev_free_idle(void *p, hipStream_t stream);

// --------------------------------------------------------------------------
// key layout: ((b << 3rb | z << 2rb | y << rb | x), rb = bits(res - 1)
// --------------------------------------------------------------------------

inline int bits_for(int64_t count)  // bits to hold values 0 .. count-1
{
    int b = 0;
    while (b < 63 && (int64_t(1) << b) < count) ++b;
    return b;
}

// Sort (key, value) pairs by the low `nbits` bits of the key, stable, LSD radix.
// The input is in the a buffers, or in the b buffers when input_in_b; the sorted
// result always ends in keys_a/vals_a (no copy when the input side is chosen by
// the parity of radix_sort_passes).  `scratch` must hold sort_scratch_bytes(n) bytes.
size_t sort_scratch_bytes(int64_t n);
int radix_sort_passes(int64_t n, int nbits);
template <typename K>
int radix_sort_pairs(K *keys_a, int32_t *vals_a, K *keys_b, int32_t *vals_b, int64_t n, int nbits,
                     void *scratch, hipStream_t stream, bool input_in_b = false);

// Exclusive scan of n uint32 values (in place allowed), or of the set-bit counts of
// n 32-bit / 64-bit words; writes the total to *total_dev if non-null.  `scratch`
// must hold scan_scratch_bytes(n) bytes; `in` and `out` must be 16-byte aligned.
// With add_back false the last pass is skipped: out[i] is then the prefix within
// i's tile of SCAN_TILE_ITEMS, and the caller adds the tile's offset, which the
// scan leaves in ((uint32_t *)scratch)[i / SCAN_TILE_ITEMS].
enum { SCAN_VALUES = 0, SCAN_POPC32 = 1, SCAN_POPC64 = 2 };
constexpr int SCAN_TILE_ITEMS = 2048;
size_t scan_scratch_bytes(int64_t n);
int exclusive_scan_u32(const uint32_t *in, uint32_t *out, int64_t n, uint32_t *total_dev,
                       void *scratch, hipStream_t stream, int input_mode = SCAN_VALUES, bool add_back = true);

// --------------------------------------------------------------------------
// bf16 helpers (bf16 values travel as uint16_t bit patterns)
// --------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f)  // round to nearest even
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float *p) { return *p; }
    static __device__ __forceinline__ float to_f32(float v) { return v; }
    static __device__ __forceinline__ float from_f32(float v) { return v; }
};
template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
    static __device__ __forceinline__ uint16_t from_f32(float v) { return f32_to_bf16(v); }
};

// --------------------------------------------------------------------------
// wave64 helpers
// --------------------------------------------------------------------------

__device__ __forceinline__ unsigned lane_id() { return __lane_id(); }
__device__ __forceinline__ uint64_t lanemask_lt() { return (uint64_t(1) << lane_id()) - 1; }

// Mask of the active lanes (valid == true) holding the same `dbits`-bit digit
// as this lane.  Must be reached by all lanes of the wave.
__device__ __forceinline__ uint64_t match_digit(uint32_t d, bool valid, int dbits)
{
    uint64_t m = __ballot(valid);
    for (int b = 0; b < dbits; ++b) {
        uint64_t bit = __ballot(valid && ((d >> b) & 1u));
        m &= ((d >> b) & 1u) ? bit : ~bit;
    }
    return m;
}

// Inclusive scan of v over a 256-thread block; `lds` holds >= 4 words.
// Returns the inclusive prefix; *total receives the block sum.
__device__ __forceinline__ uint32_t block_incl_scan256(uint32_t v, uint32_t *lds, uint32_t *total)
{
    const unsigned lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t y = __shfl_up(x, off, 64);
        if (lane >= (unsigned)off) x += y;
    }
    if (lane == 63) lds[wave] = x;
    __syncthreads();
    uint32_t before = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t t = lds[w];
        before += (w < (int)wave) ? t : 0u;
        sum += t;
    }
    __syncthreads();
    *total = sum;
    return x + before;
}

// Group windows: per group of 32 consecutive sorted voxels, for each of the 9
// (dz, dy) rows the first (ints 0-8) and last (ints 9-17) sorted position its
// neighbours in that row occupy; an empty row holds (GWIN_NONE, -1).
constexpr int GWIN_INTS = 18;
constexpr int32_t GWIN_NONE = 0x7fffffff;

// Neighbour rows of the rulebook, NBR_INTS int32 per sorted voxel.  For a (dz, dy)
// row d = 3 (dz + 1) + (dy + 1), the voxel's neighbours at x - 1, x, x + 1 are keys
// adjacent in sorted order, so their sorted positions are consecutive: ints 0-8
// hold the position of each row's first present cell, int 9 the presence bits
// (bit 3 d + j: cell x - 1 + j of row d exists).  The neighbour of tap k = 3 d + j
// sits at first[d] + (present cells of the row before j).  40 bytes per voxel
// instead of 108 for the 27 positions spelled out.
constexpr int NBR_INTS = 10;

// Sorted position of tap k's neighbour, or -1.
__device__ __forceinline__ int32_t nbr_at(const int32_t *row, int k)
{
    const int d = k / 3, j = k - 3 * d;
    const uint32_t m = ((uint32_t)row[9] >> (3 * d)) & 7u;
    return ((m >> j) & 1u) ? row[d] + (int32_t)__popc(m & ((1u << j) - 1u)) : -1;
}

// The same from registers: first positions of rows d0 .. d0 + 4 and the presence bits
// (k compile-time: ALU only).
template <int D0>
__device__ __forceinline__ int32_t nbr_at_reg(const int32_t (&first)[5], uint32_t mask, int k)
{
    const int d = k / 3, j = k - 3 * d;
    const uint32_t m = (mask >> (3 * d)) & 7u;
    return ((m >> j) & 1u) ? first[d - D0] + (int32_t)__popc(m & ((1u << j) - 1u)) : -1;
}

// The row form of 27 sorted positions (-1 = absent).
__device__ __forceinline__ void nbr_pack(const int32_t (&p)[27], int32_t (&r)[NBR_INTS])
{
    uint32_t mask = 0;
#pragma unroll
    for (int d = 0; d < 9; ++d) {
        const int32_t a = p[3 * d], b = p[3 * d + 1], c = p[3 * d + 2];
        r[d] = a >= 0 ? a : (b >= 0 ? b : (c >= 0 ? c : 0));
        mask |= (a >= 0 ? 1u : 0u) << (3 * d);
        mask |= (b >= 0 ? 2u : 0u) << (3 * d);
        mask |= (c >= 0 ? 4u : 0u) << (3 * d);
    }
    r[9] = (int32_t)mask;
}

}  // namespace sc

// Rulebook: library-owned device memory for one coordinate set.  Everything is
// indexed by sorted position s (C order of the packed key).
struct submconv_rulebook {
    int64_t n;
    int32_t res;
    int32_t batch;
    int32_t rb;         // bits per spatial axis in the key
    int32_t nbits;      // significant key bits
    int32_t key_bytes;  // 4 or 8
    int32_t device;
    int64_t taps;       // P: present entries of the table
    int64_t ngroups;    // groups of 32 sorted voxels
    void *block;        // single allocation holding the arrays below
    size_t block_bytes; // its size
    void *keys;         // sorted keys [n]
    int32_t *perm;      // sorted position -> input row [n]
    int32_t *nbr_sp;    // [n,NBR_INTS]: neighbour rows by sorted position (see NBR_INTS; padded allocation)
    int32_t *gwin;      // [ngroups,18]: group row windows (see mapbuild.hip)
    int32_t *nbr_in;    // [n,27] input-order table of input rows, built on first request (or null)
    int32_t *plan;      // staging plan of the windowed forward kernel (see conv_win.hip)
};
