// Device radix sort of (key, row) pairs and device exclusive scan.
//
// LSD radix sort over only the significant key bits (a coordinate key of a
// 512^3 grid has 27), at most 8 bits per pass.  Each pass is three kernels:
//   hist    - per-tile digit counts (wave-aggregated LDS atomics),
//   scan    - per-digit exclusive scan over tiles + digit totals,
//   scatter - stable rank inside the tile (wave ballots), local sort in LDS,
//             then coalesced writes of each digit's run to its global slot.
// No kernel waits on another block, so no pass can deadlock.
#include "common.h"

namespace sc {

constexpr int SORT_THREADS = 256;
constexpr int SORT_ITEMS = 8;
constexpr int SORT_TILE = SORT_THREADS * SORT_ITEMS;
constexpr int MAX_DIGIT_BITS = 8;
constexpr int MAX_BINS = 1 << MAX_DIGIT_BITS;

static inline int64_t sort_tiles(int64_t n) { return (n + SORT_TILE - 1) / SORT_TILE; }

size_t sort_scratch_bytes(int64_t n)
{
    // hist + offs ([bins][tiles] each) + bin totals
    return (size_t)(2 * MAX_BINS * sort_tiles(n) + MAX_BINS) * sizeof(uint32_t) + 256;
}

template <typename K>
__global__ __launch_bounds__(SORT_THREADS) void k_sort_hist(const K *__restrict__ keys, int64_t n,
                                                            int shift, int dbits,
                                                            uint32_t *__restrict__ hist, int ntiles)
{
    __shared__ uint32_t cnt[MAX_BINS];
    const int bins = 1 << dbits;
    for (int t = threadIdx.x; t < bins; t += SORT_THREADS) cnt[t] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * SORT_TILE;
    for (int it = 0; it < SORT_ITEMS; ++it) {
        const int64_t i = base + it * SORT_THREADS + threadIdx.x;
        const bool valid = i < n;
        const uint32_t d = valid ? (uint32_t)(keys[i] >> shift) & (uint32_t)(bins - 1) : 0u;
        const uint64_t peers = match_digit(d, valid, dbits);
        if (valid && (peers & lanemask_lt()) == 0) atomicAdd(&cnt[d], (uint32_t)__popcll(peers));
    }
    __syncthreads();
    for (int t = threadIdx.x; t < bins; t += SORT_THREADS) hist[(size_t)t * ntiles + blockIdx.x] = cnt[t];
}

// One block per digit: exclusive scan of hist[d][0..ntiles) into offs, total into bin_total[d].
__global__ __launch_bounds__(256) void k_sort_scan(const uint32_t *__restrict__ hist,
                                                   uint32_t *__restrict__ offs,
                                                   uint32_t *__restrict__ bin_total, int ntiles)
{
    __shared__ uint32_t lds[4];
    const uint32_t *h = hist + (size_t)blockIdx.x * ntiles;
    uint32_t *o = offs + (size_t)blockIdx.x * ntiles;
    uint32_t carry = 0;
    for (int base = 0; base < ntiles; base += 256) {
        const int i = base + threadIdx.x;
        const uint32_t v = i < ntiles ? h[i] : 0u;
        uint32_t total;
        const uint32_t incl = block_incl_scan256(v, lds, &total);
        if (i < ntiles) o[i] = carry + incl - v;
        carry += total;
    }
    if (threadIdx.x == 0) bin_total[blockIdx.x] = carry;
}

template <typename K>
__global__ __launch_bounds__(SORT_THREADS) void k_sort_scatter(
    const K *__restrict__ kin, const int32_t *__restrict__ vin, K *__restrict__ kout,
    int32_t *__restrict__ vout, int64_t n, int shift, int dbits, const uint32_t *__restrict__ hist,
    const uint32_t *__restrict__ offs, const uint32_t *__restrict__ bin_total, int ntiles)
{
    __shared__ K s_keys[SORT_TILE];
    __shared__ int32_t s_vals[SORT_TILE];
    __shared__ uint32_t s_gbase[MAX_BINS];  // global position of local position 0 of digit d
    __shared__ uint32_t s_lbase[MAX_BINS];  // start of digit d inside the locally sorted tile
    __shared__ uint32_t s_run[MAX_BINS];    // digit d items placed so far
    __shared__ uint32_t s_wcnt[SORT_THREADS / 64][MAX_BINS];
    __shared__ uint32_t s_scan[4];

    const int bins = 1 << dbits;
    const int tid = threadIdx.x, wave = tid >> 6;
    const uint32_t dmask = (uint32_t)(bins - 1);

    // digit bases: bins <= 256 = one digit per thread
    const uint32_t bt = tid < bins ? bin_total[tid] : 0u;
    const uint32_t hc = tid < bins ? hist[(size_t)tid * ntiles + blockIdx.x] : 0u;
    uint32_t tot;
    const uint32_t bt_ex = block_incl_scan256(bt, s_scan, &tot) - bt;
    const uint32_t hc_ex = block_incl_scan256(hc, s_scan, &tot) - hc;
    if (tid < bins) {
        s_gbase[tid] = bt_ex + offs[(size_t)tid * ntiles + blockIdx.x] - hc_ex;
        s_lbase[tid] = hc_ex;
        s_run[tid] = 0;
#pragma unroll
        for (int w = 0; w < SORT_THREADS / 64; ++w) s_wcnt[w][tid] = 0;
    }
    __syncthreads();

    const int64_t base = (int64_t)blockIdx.x * SORT_TILE;
    const int tile_n = (int)((n - base) < SORT_TILE ? (n - base) : SORT_TILE);
    for (int it = 0; it < SORT_ITEMS; ++it) {
        const int li = it * SORT_THREADS + tid;
        const bool valid = li < tile_n;
        const K key = valid ? kin[base + li] : K(0);
        const int32_t val = valid ? vin[base + li] : 0;
        const uint32_t d = (uint32_t)(key >> shift) & dmask;
        const uint64_t peers = match_digit(d, valid, dbits);
        const uint32_t rank = (uint32_t)__popcll(peers & lanemask_lt());
        if (valid && rank == 0) s_wcnt[wave][d] = (uint32_t)__popcll(peers);
        __syncthreads();
        if (tid < bins) {  // counts -> exclusive offsets per wave, in wave order (stable)
            uint32_t run = s_run[tid];
#pragma unroll
            for (int w = 0; w < SORT_THREADS / 64; ++w) {
                const uint32_t c = s_wcnt[w][tid];
                s_wcnt[w][tid] = run;
                run += c;
            }
            s_run[tid] = run;
        }
        __syncthreads();
        if (valid) {
            const uint32_t pos = s_lbase[d] + s_wcnt[wave][d] + rank;
            s_keys[pos] = key;
            s_vals[pos] = val;
        }
        __syncthreads();
        if (tid < bins) {
#pragma unroll
            for (int w = 0; w < SORT_THREADS / 64; ++w) s_wcnt[w][tid] = 0;
        }
        __syncthreads();
    }
    for (int p = tid; p < tile_n; p += SORT_THREADS) {
        const K key = s_keys[p];
        const uint32_t d = (uint32_t)(key >> shift) & dmask;
        const size_t g = (size_t)(uint32_t)(s_gbase[d] + (uint32_t)p);
        kout[g] = key;
        vout[g] = s_vals[p];
    }
}

int radix_sort_passes(int64_t n, int nbits)
{
    if (n <= 1 || nbits <= 0) return 0;
    return (nbits + MAX_DIGIT_BITS - 1) / MAX_DIGIT_BITS;
}

template <typename K>
int radix_sort_pairs(K *keys_a, int32_t *vals_a, K *keys_b, int32_t *vals_b, int64_t n, int nbits,
                     void *scratch, hipStream_t stream, bool input_in_b)
{
    const int npass = radix_sort_passes(n, nbits);
    if (npass == 0) {
        if (input_in_b && n > 0) {
            SC_HIP(hipMemcpyAsync(keys_a, keys_b, (size_t)n * sizeof(K), hipMemcpyDeviceToDevice, stream));
            SC_HIP(hipMemcpyAsync(vals_a, vals_b, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToDevice, stream));
        }
        return SUBMCONV_OK;
    }
    const int dbits = (nbits + npass - 1) / npass;
    const int bins = 1 << dbits;
    const int ntiles = (int)sort_tiles(n);
    uint32_t *hist = (uint32_t *)scratch;
    uint32_t *offs = hist + (size_t)MAX_BINS * ntiles;
    uint32_t *bin_total = offs + (size_t)MAX_BINS * ntiles;
    K *src_k = input_in_b ? keys_b : keys_a, *dst_k = input_in_b ? keys_a : keys_b;
    int32_t *src_v = input_in_b ? vals_b : vals_a, *dst_v = input_in_b ? vals_a : vals_b;
    for (int p = 0; p < npass; ++p) {
        const int shift = p * dbits;
        hipLaunchKernelGGL(k_sort_hist<K>, dim3(ntiles), dim3(SORT_THREADS), 0, stream, src_k, n,
                           shift, dbits, hist, ntiles);
        SC_LAUNCHED("sort_hist");
        hipLaunchKernelGGL(k_sort_scan, dim3(bins), dim3(256), 0, stream, hist, offs, bin_total,
                           ntiles);
        SC_LAUNCHED("sort_scan");
        hipLaunchKernelGGL(k_sort_scatter<K>, dim3(ntiles), dim3(SORT_THREADS), 0, stream, src_k,
                           src_v, dst_k, dst_v, n, shift, dbits, hist, offs, bin_total, ntiles);
        SC_LAUNCHED("sort_scatter");
        K *tk = src_k; src_k = dst_k; dst_k = tk;
        int32_t *tv = src_v; src_v = dst_v; dst_v = tv;
    }
    if (src_k != keys_a) {  // the pass count left the result in the b buffers
        SC_HIP(hipMemcpyAsync(keys_a, src_k, (size_t)n * sizeof(K), hipMemcpyDeviceToDevice, stream));
        SC_HIP(hipMemcpyAsync(vals_a, src_v, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToDevice,
                              stream));
    }
    return SUBMCONV_OK;
}

template int radix_sort_pairs<uint32_t>(uint32_t *, int32_t *, uint32_t *, int32_t *, int64_t, int,
                                        void *, hipStream_t, bool);
template int radix_sort_pairs<uint64_t>(uint64_t *, int32_t *, uint64_t *, int32_t *, int64_t, int,
                                        void *, hipStream_t, bool);

// --------------------------------------------------------------------------
// exclusive scan of uint32 (tiles of 2048, then the tile sums, then add back)
// --------------------------------------------------------------------------

constexpr int SCAN_ITEMS = 8;
constexpr int SCAN_TILE = 256 * SCAN_ITEMS;
static_assert(SCAN_TILE == SCAN_TILE_ITEMS, "tile size exported in common.h");

size_t scan_scratch_bytes(int64_t n)
{
    const int64_t tiles = (n + SCAN_TILE - 1) / SCAN_TILE;
    return (size_t)(tiles + 1) * sizeof(uint32_t) + 256;
}

// Per tile: exclusive scan in place into `out`, tile sum into sums[tile].  With
// POPC the scanned value of an input word is its number of set bits.
// MODE 0: the values themselves; 1: set bits of 32-bit words; 2: set bits of
// 64-bit words (`in` then points at n 64-bit words).
template <int MODE>
__global__ __launch_bounds__(256) void k_scan_tiles(const uint32_t *__restrict__ in,
                                                    uint32_t *__restrict__ out, int64_t n,
                                                    uint32_t *__restrict__ sums)
{
    __shared__ uint32_t lds[4];
    const int64_t base = (int64_t)blockIdx.x * SCAN_TILE + (int64_t)threadIdx.x * SCAN_ITEMS;
    // A thread's items are contiguous: a full run moves as 16-byte loads and stores
    // (a thread's first item is 32- or 64-byte aligned: base is a multiple of 8).
    const bool full = base + SCAN_ITEMS <= n;
    uint32_t v[SCAN_ITEMS];
    uint32_t local = 0;
    if (MODE == 2 && full) {
        const ulonglong2 *src = (const ulonglong2 *)((const uint64_t *)in + base);
#pragma unroll
        for (int h = 0; h < SCAN_ITEMS / 2; ++h) {
            const ulonglong2 x = src[h];
            v[2 * h] = (uint32_t)__popcll(x.x);
            v[2 * h + 1] = (uint32_t)__popcll(x.y);
        }
    } else if (MODE != 2 && full) {
        const uint4 *src = (const uint4 *)(in + base);
#pragma unroll
        for (int h = 0; h < SCAN_ITEMS / 4; ++h) {
            const uint4 x = src[h];
            v[4 * h] = MODE == 1 ? (uint32_t)__popc(x.x) : x.x;
            v[4 * h + 1] = MODE == 1 ? (uint32_t)__popc(x.y) : x.y;
            v[4 * h + 2] = MODE == 1 ? (uint32_t)__popc(x.z) : x.z;
            v[4 * h + 3] = MODE == 1 ? (uint32_t)__popc(x.w) : x.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < SCAN_ITEMS; ++e) {
            if (MODE == 2) {
                const uint64_t x = (base + e < n) ? ((const uint64_t *)in)[base + e] : 0ull;
                v[e] = (uint32_t)__popcll(x);
            } else {
                const uint32_t x = (base + e < n) ? in[base + e] : 0u;
                v[e] = MODE == 1 ? (uint32_t)__popc(x) : x;
            }
        }
    }
#pragma unroll
    for (int e = 0; e < SCAN_ITEMS; ++e) local += v[e];
    uint32_t total;
    const uint32_t incl = block_incl_scan256(local, lds, &total);
    uint32_t run = incl - local;
    uint32_t o[SCAN_ITEMS];
#pragma unroll
    for (int e = 0; e < SCAN_ITEMS; ++e) {
        o[e] = run;
        run += v[e];
    }
    if (full) {
        uint4 *dst = (uint4 *)(out + base);
#pragma unroll
        for (int h = 0; h < SCAN_ITEMS / 4; ++h) dst[h] = make_uint4(o[4 * h], o[4 * h + 1], o[4 * h + 2], o[4 * h + 3]);
    } else {
#pragma unroll
        for (int e = 0; e < SCAN_ITEMS; ++e)
            if (base + e < n) out[base + e] = o[e];
    }
    if (threadIdx.x == 0) sums[blockIdx.x] = total;
}

// Single block: exclusive scan of the tile sums; grand total to *total.
__global__ __launch_bounds__(256) void k_scan_sums(uint32_t *__restrict__ sums, int64_t ntiles,
                                                   uint32_t *__restrict__ total_out)
{
    __shared__ uint32_t lds[4];
    uint32_t carry = 0;
    for (int64_t base = 0; base < ntiles; base += 256) {
        const int64_t i = base + threadIdx.x;
        const uint32_t v = i < ntiles ? sums[i] : 0u;
        uint32_t total;
        const uint32_t incl = block_incl_scan256(v, lds, &total);
        if (i < ntiles) sums[i] = carry + incl - v;
        carry += total;
    }
    if (threadIdx.x == 0 && total_out) *total_out = carry;
}

__global__ __launch_bounds__(256) void k_scan_add(uint32_t *__restrict__ out, int64_t n,
                                                  const uint32_t *__restrict__ sums)
{
    const uint32_t add = sums[blockIdx.x];
    const int64_t base = (int64_t)blockIdx.x * SCAN_TILE;
    for (int e = threadIdx.x; e < SCAN_TILE; e += 256)
        if (base + e < n) out[base + e] += add;
}

int exclusive_scan_u32(const uint32_t *in, uint32_t *out, int64_t n, uint32_t *total_dev,
                       void *scratch, hipStream_t stream, int input_mode, bool add_back)
{
    if (n <= 0) {
        if (total_dev) SC_HIP(hipMemsetAsync(total_dev, 0, sizeof(uint32_t), stream));
        return SUBMCONV_OK;
    }
    const int64_t tiles = (n + SCAN_TILE - 1) / SCAN_TILE;
    uint32_t *sums = (uint32_t *)scratch;
    if (input_mode == SCAN_POPC64)
        hipLaunchKernelGGL(k_scan_tiles<2>, dim3((unsigned)tiles), dim3(256), 0, stream, in, out, n, sums);
    else if (input_mode == SCAN_POPC32)
        hipLaunchKernelGGL(k_scan_tiles<1>, dim3((unsigned)tiles), dim3(256), 0, stream, in, out, n, sums);
    else
        hipLaunchKernelGGL(k_scan_tiles<0>, dim3((unsigned)tiles), dim3(256), 0, stream, in, out, n, sums);
    SC_LAUNCHED("scan_tiles");
    hipLaunchKernelGGL(k_scan_sums, dim3(1), dim3(256), 0, stream, sums, tiles, total_dev);
    SC_LAUNCHED("scan_sums");
    if (tiles > 1 && add_back) {
        hipLaunchKernelGGL(k_scan_add, dim3((unsigned)tiles), dim3(256), 0, stream, out, n, sums);
        SC_LAUNCHED("scan_add");
    }
    return SUBMCONV_OK;
}

}  // namespace sc
