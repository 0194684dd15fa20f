// Windowed forward kernel: a tile's whole neighbourhood staged once in LDS.
//
// The convolution (lato.2_mrp_mlx working notes, "Key facts" and commit
// summary) is the same as in conv.hip:
//   out[i, o] = bias[o] + sum_k sum_c W[o, k', c] * feats[nbr[i, k], c].
// Gathering a 64-byte feature row per (voxel, tap) through the vector-memory
// path is bound by per-cache-line work, not bytes: a random-row gather that
// misses L1 moves only a fraction of what LDS moves for the same pattern.  So
// this kernel stages each tile's neighbour rows in LDS once, using what the map
// builder records: sorted voxels' neighbours in one (dz, dy) row lie in a narrow
// window of sorted positions, and the windows of a tile's 9 rows merge into a
// few ranges.  A neighbour's LDS slot is then its sorted position plus a
// per-row constant, so no search and no deduplication is needed.
//
// Tiles of 128 sorted voxels; one persistent block per CU, 8 waves (two per
// SIMD).  Waves w and w + 4 compute the same 32-voxel column of the tile, over
// taps 0-13 and 14-26, and add their partial sums through LDS at the end.
//   * each wave's weight taps sit in registers for the whole kernel (MFMA A
//     operand, out^T = W_k . F_k^T, rows = output channels);
//   * double-buffered LDS: while a tile is computed, the next tile's rows and
//     neighbour-table block are copied in by direct global->LDS loads, and the
//     sorted->input row numbers of the tile after that are fetched;
//   * rows are stored as four 16-byte chunks with the chunk order XOR-swizzled
//     by the slot, so the 32 rows a B-operand read touches spread over the
//     LDS banks;
//   * a tile whose merged windows exceed the buffer is computed with direct
//     global gathers instead (rare on surface data);
//   * tiles are split among the 8 XCDs in contiguous runs (a workgroup's XCD is
//     its id mod 8), so neighbouring tiles share an L2.
// Accumulation is fp32; the bf16 output is one rounding of the fp32 sum.
#include <type_traits>
#include <utility>

#include "common.h"
#include "winplan.h"

namespace sc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));  // converted with round-to-nearest-even
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

__device__ uint4 g_win_zero[16] = {};  // 256 bytes of zeros: padding slots and missing rows

// Plans from the group windows (the builds that do not compute them in their
// resolve): a team of 16 lanes per tile, lane q < 9 taking (dz, dy) row q, the union
// of its window over the tile's groups (plan_tile_team, winplan.h).  The block's
// records are assembled in LDS and written as one contiguous run.  The first
// PLAN_TAP_BLOCKS blocks also sum the per-block present counts of the resolve
// (blk_taps, when given) into st->taps.
constexpr int PLAN_GPT = WIN_TILE / 32;              // groups per tile
constexpr int PLAN_THREADS = 256;
constexpr int PLAN_TILES = PLAN_THREADS / 16;        // tiles per block
constexpr int PLAN_TAP_BLOCKS = 64;
__global__ __launch_bounds__(PLAN_THREADS) void k_win_plan(const int32_t *__restrict__ gwin, int64_t ngroups,
                                                           int64_t ntiles, int cap, int32_t *__restrict__ plan,
                                                           const uint32_t *__restrict__ blk_taps, int64_t nblk,
                                                           DevStatus *st)
{
    __shared__ __attribute__((aligned(16))) int32_t s_rec[PLAN_TILES * PLAN_INTS];
    const int tid = threadIdx.x, q = tid & 15, team = tid >> 4;
    const int64_t t0 = (int64_t)blockIdx.x * PLAN_TILES, t = t0 + team;
    if (blk_taps && blockIdx.x < PLAN_TAP_BLOCKS) {
        const int64_t stride = (int64_t)min((int64_t)gridDim.x, (int64_t)PLAN_TAP_BLOCKS) * PLAN_THREADS;
        unsigned long long taps = 0;
        for (int64_t b = (int64_t)blockIdx.x * PLAN_THREADS + tid; b < nblk; b += stride) taps += blk_taps[b];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) taps += __shfl_xor(taps, off, 64);
        if ((tid & 63) == 0 && taps) atomicAdd(&st->taps, taps);
    }

    // row q's window over the tile's groups (groups past ngroups are empty)
    int32_t lo = GWIN_NONE, hi = -1;
    if (t < ntiles && q < 9) {
        int32_t wl[PLAN_GPT], wh[PLAN_GPT];
#pragma unroll
        for (int g = 0; g < PLAN_GPT; ++g) {
            const int64_t gi = min(t * PLAN_GPT + g, ngroups - 1);
            wl[g] = gwin[gi * GWIN_INTS + q];
            wh[g] = gwin[gi * GWIN_INTS + 9 + q];
        }
#pragma unroll
        for (int g = 0; g < PLAN_GPT; ++g) {
            if (t * PLAN_GPT + g < ngroups && wh[g] >= 0) {
                lo = min(lo, wl[g]);
                hi = max(hi, wh[g]);
            }
        }
    }
    plan_tile_team(lo, hi, q, cap, s_rec + team * PLAN_INTS);
    __syncthreads();
    const int rows = (int)min((int64_t)PLAN_TILES, ntiles - t0);
    if (tid < rows * (PLAN_INTS / 4))
        ((int4 *)(plan + t0 * PLAN_INTS))[tid] = ((const int4 *)s_rec)[tid];
}

// ---------------------------------------------------------------------------
// the kernel (bf16, Cin = Cout = 32)
// ---------------------------------------------------------------------------

constexpr int W32_ROW = 64;                                   // bytes per staged row
constexpr int W32_TBL = 5 * 1024 + 512;                       // neighbour rows of the tile (5120 B)
                                                              // then the tile's 128 sort-order row numbers
constexpr int W32_PERM = WIN_SLOTS * 64 + 5 * 1024;           // offset of those row numbers
constexpr int W32_BUF = WIN_SLOTS * W32_ROW + W32_TBL;        // one buffer
constexpr int W32_LDS = 2 * W32_BUF;                          // 142336 B, two buffers
constexpr int W32_RED = 4 * 4 * 64 * 16;                       // partial sums of the second tap half
static_assert(W32_LDS + W32_RED + 32 * 4 <= 160 * 1024, "LDS budget (buffers, partial sums, bias)");
static_assert(WIN_TILE * NBR_INTS * 4 + 512 <= W32_TBL, "table block");

__device__ __forceinline__ int w32_chunk_addr(int slot, int chunk)  // byte offset of a row chunk
{
    return slot * W32_ROW + ((chunk ^ ((slot >> 1) & 3)) << 4);
}

__device__ __forceinline__ int plan_get(int pv, int idx) { return __builtin_amdgcn_readlane(pv, idx); }

constexpr int W32_WAVES = 8;   // two per SIMD; waves w and w+4 share a 32-voxel column
constexpr int W32_CHUNKS = 2;  // 64-slot chunks of a tile's row numbers per wave: wave + 8c
static_assert(W32_WAVES * W32_CHUNKS * 64 >= WIN_SLOTS, "row-number chunks cover the buffer");

// A copy instruction puts lane l's 16 bytes at slot 16i + l/4, position l%4; the
// position holds chunk (l%4) ^ ((slot >> 1) & 3) = (l%4) ^ ((l >> 3) & 3).
__device__ __forceinline__ int w32_lane_chunk(int lane) { return (lane & 3) ^ ((lane >> 3) & 3); }

// The ranges of a tile's plan in registers: slots from off[r] hold sorted
// positions slot + base[r].
struct W32Ranges {
    int R, nr;
    int off[9], base[9];
};
__device__ __forceinline__ W32Ranges w32_ranges(int pv)
{
    W32Ranges g;
    g.R = plan_get(pv, 0);
    g.nr = plan_get(pv, 1);
#pragma unroll
    for (int r = 0; r < 9; ++r) {
        g.off[r] = plan_get(pv, 11 + r);
        g.base[r] = plan_get(pv, 2 + r) - g.off[r];
    }
    return g;
}

// Input row of `slot` (slots < R): one lane per slot.
// The load is unconditional (a slot past R reads a clamped position whose value the
// copy ignores) and its value is not inspected here, so it is not waited for until
// the copies of its tile use it.
__device__ __forceinline__ int32_t w32_row_of(const int32_t *__restrict__ perm, int64_t n, const W32Ranges &g,
                                              int slot)
{
    int32_t b = g.base[0];
#pragma unroll
    for (int q = 1; q < 9; ++q) {
        if (q >= g.nr) break;
        b = slot >= g.off[q] ? g.base[q] : b;
    }
    const int32_t pos = b + slot;
    return perm[pos < 0 ? 0 : (pos >= (int32_t)n ? (int32_t)n - 1 : pos)];
}

// Row copy `item` = 4c + q of this wave: slots 64k + 16q .. +15 of chunk k = wave + 8c.
// rid[item] holds, in lane l, the input row of slot 64k + 16q + l/4.  The rows come
// through a buffer resource over the features (n * 64 bytes): a row is a 32-bit
// byte offset, and a missing row an offset past the end, which reads zeros.
__device__ __forceinline__ void w32_copy_rows(char *buf, __amdgpu_buffer_rsrc_t frs, int64_t n, int R,
                                              int32_t rid, int item, int wave, int lane, int lchunk)
{
    const int k = wave + W32_WAVES * (item >> 2);
    const int slot0 = 64 * k + 16 * (item & 3);
    if (slot0 >= R) return;
    const int slot = slot0 + (lane >> 2);
    const uint32_t voff = slot < R && (uint32_t)rid < (uint32_t)n ? (uint32_t)rid * W32_ROW + (uint32_t)lchunk * 16u
                                                                  : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(frs, (lds_void *)(buf + slot0 * W32_ROW), 16, voff, 0, 0, 0);
}

// Copies of a tile's neighbour-table block (whole 1-KB copies; the table
// allocation is padded by 1 KB) and of its 128 output row numbers perm[s0 ..]
// (4 bytes per lane; entries past n read the table allocation that follows perm
// and are never used).
__device__ __forceinline__ void w32_copy_table(char *buf, const int32_t *__restrict__ nbr_sp,
                                               const int32_t *__restrict__ perm, int64_t n, int64_t tile,
                                               int wave, int lane)
{
    const int64_t s0 = tile * WIN_TILE;
    const int64_t cnt = (n - s0) < WIN_TILE ? (n - s0) : WIN_TILE;
    const int nt = (int)((cnt * NBR_INTS * 4 + 1023) >> 10);
    const char *tb = (const char *)(nbr_sp + s0 * NBR_INTS);
    for (int i = wave; i < nt; i += W32_WAVES)
        __builtin_amdgcn_global_load_lds((gbl_void *)(tb + i * 1024 + lane * 16),
                                         (lds_void *)(buf + WIN_SLOTS * W32_ROW + i * 1024), 16, 0, 0);
    if (wave == W32_WAVES - 1) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
            __builtin_amdgcn_global_load_lds((gbl_void *)(perm + s0 + 64 * h + lane),
                                             (lds_void *)(buf + W32_PERM + 256 * h), 4, 0, 0);
    }
}

// Spread the row numbers (one per lane and slot) to the copy lanes (four per slot).
__device__ __forceinline__ void w32_expand(const int32_t (&rows)[W32_CHUNKS], int32_t (&rid)[4 * W32_CHUNKS],
                                           int lane)
{
#pragma unroll
    for (int c = 0; c < W32_CHUNKS; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) rid[4 * c + q] = __shfl(rows[c], 16 * q + (lane >> 2), 64);
}

// Barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// global loads (the next tile's copies stay in flight across it).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ void w32_mfma(floatx16 &acc, const uint4 &a, const uint4 &b)
{
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  acc, 0, 0, 0);
}

template <int J> using w32_item = std::integral_constant<int, J>;
constexpr int W32_ITEMS = 10;  // side-work items per tile (see the kernel)

// f(w32_item<I>{}), ..., f(w32_item<N - 1>{}) with compile-time indices
template <int I, int N, typename F>
__device__ __forceinline__ void w32_unroll(F &&f)
{
    if constexpr (I < N) {
        f(w32_item<I>{});
        w32_unroll<I + 1, N>(f);
    }
}

// Taps K0 .. K0 + NK - 1 of this lane's voxel from the staged rows, with the
// tile's side work (copies for the next tiles, stores of the previous one)
// issued between the MFMAs.  tbl: the voxel's neighbour row in LDS (decoded per
// tap into a sorted position); delta from the plan; ok: the voxel exists.  Row reads run
// PF taps ahead of their MFMAs.  Chunk 2 + kh sits at the chunk-kh address XOR
// 32 (the swizzle flips bit 1 of the position, and 2 + kh = kh ^ 2).
template <int K0, int NK, typename Side>
__device__ __forceinline__ void w32_taps_lds(floatx16 &acc, const char *cur, const int32_t *tbl, const int (&delta)[9],
                                             bool ok, int kh, const uint4 (&wf)[14][2], Side &&side)
{
    constexpr int PF = 1;
    constexpr int D0 = K0 / 3;  // this tap half's rows are D0 .. D0 + 4
    // Per (dz,dy) row, once per tile: the LDS slot of its first present cell (its
    // sorted position plus the plan's offset) and its presence bits (none when the
    // voxel is not valid).  A tap is then a bit test, at most a popcount, a clamp
    // and the swizzled address: the tap loop is bound by VALU issue, not by MFMA.
    int32_t rslot[5];
    uint32_t rbits[5];
    const uint32_t mask = ok ? (uint32_t)tbl[9] : 0u;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        rslot[i] = D0 + i < 9 ? tbl[D0 + i] + delta[D0 + i] : 0;
        rbits[i] = D0 + i < 9 ? (mask >> (3 * (D0 + i))) & 7u : 0u;
    }
    const int kh16 = kh << 4;
    uint4 b[PF + 1][2];
    auto prep = [&](int j) {
        const int d = (K0 + j) / 3 - D0, jj = (K0 + j) % 3;
        const uint32_t m = rbits[d];
        const int32_t off = jj == 0 ? 0 : (jj == 1 ? (int32_t)(m & 1u) : (int32_t)__popc(m & 3u));
        // a missing neighbour reads the zero slot; an out-of-range slot (not produced
        // by a consistent table and plan) is clamped to it
        const uint32_t slot = ((m >> jj) & 1u) ? min((uint32_t)(rslot[d] + off), (uint32_t)WIN_CAP) : (uint32_t)WIN_CAP;
        const int addr = (int)(slot * W32_ROW) | ((((int)slot << 3) & 0x30) ^ kh16);  // w32_chunk_addr(slot, kh)
        b[j % (PF + 1)][0] = *(const uint4 *)(cur + addr);
        b[j % (PF + 1)][1] = *(const uint4 *)(cur + (addr ^ 32));
    };
#pragma unroll
    for (int j = 0; j < PF; ++j) prep(j);
    auto one = [&](auto jc) {
        constexpr int j = decltype(jc)::value;
        if constexpr (j + PF < NK) prep(j + PF);
        if constexpr (j < W32_ITEMS) side(jc);
        __builtin_amdgcn_sched_barrier(0);  // keep the reads and the side work ahead of the MFMAs
        w32_mfma(acc, wf[j][0], b[j % (PF + 1)][0]);
        w32_mfma(acc, wf[j][1], b[j % (PF + 1)][1]);
        __builtin_amdgcn_sched_barrier(0);
    };
    w32_unroll<0, NK>(one);
    w32_unroll<NK, W32_ITEMS>(side);
}

// The same taps gathered from global memory (a tile whose neighbourhood did not fit);
// the side work goes first.
template <int K0, int NK, typename Side>
__device__ __forceinline__ void w32_taps_global(floatx16 &acc, const uint16_t *__restrict__ feats,
                                                const int32_t *__restrict__ perm, int64_t n, const int32_t *tbl,
                                                bool ok, int kh, const uint4 (&wf)[14][2], Side &&side)
{
    w32_unroll<0, W32_ITEMS>(side);
#pragma unroll
    for (int j = 0; j < NK; ++j) {
        const int32_t e = nbr_at(tbl, K0 + j);
        const int32_t r = (ok && e >= 0 && e < n) ? perm[e] : -1;
        uint4 b0 = make_uint4(0, 0, 0, 0), b1 = b0;
        if ((uint32_t)r < (uint64_t)n) {
            b0 = *(const uint4 *)(feats + (int64_t)r * 32 + 8 * kh);
            b1 = *(const uint4 *)(feats + (int64_t)r * 32 + 16 + 8 * kh);
        }
        w32_mfma(acc, wf[j][0], b0);
        w32_mfma(acc, wf[j][1], b1);
    }
}

__global__ __launch_bounds__(512, 2) void k_conv_win32(const uint16_t *__restrict__ feats,
                                                       const uint16_t *__restrict__ weight,
                                                       const float *__restrict__ bias,
                                                       const int32_t *__restrict__ nbr_sp,
                                                       const int32_t *__restrict__ perm,
                                                       const int32_t *__restrict__ plan,
                                                       uint16_t *__restrict__ out, int64_t n,
                                                       int64_t ntiles, int flip)
{
    // two buffers as two objects: the compiler tracks the direct-to-LDS copies per
    // object, so reads of one buffer need not wait for copies into the other
    __shared__ __attribute__((aligned(1024))) char buf0[W32_BUF];
    __shared__ __attribute__((aligned(1024))) char buf1[W32_BUF];
    // the bias, read once: a global load in the reduction waits for every copy in flight
    __shared__ __attribute__((aligned(16))) float s_bias[32];
    // the second tap half's partial sums (its own buffer: writing them needs no wait for
    // the other waves to finish reading the current rows)
    __shared__ __attribute__((aligned(16))) float4 s_red[W32_RED / 16];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, kh = lane >> 5;
    const int cb = wave & 3, th = wave >> 2;  // column block, tap half (taps 0-13 or 14-26)
    const int lchunk = w32_lane_chunk(lane);
    const __amdgpu_buffer_rsrc_t frs = __builtin_amdgcn_make_buffer_rsrc((void *)feats, 0, (int)(n * W32_ROW), 0x00020000);

    // tiles of this block: the XCD's contiguous run, dealt round-robin to its blocks
    const int xcd = blockIdx.x & 7, bpx = gridDim.x >> 3, jb = blockIdx.x >> 3;
    const int64_t t_begin = ntiles * xcd / 8, t_end = ntiles * (xcd + 1) / 8;
    const int64_t first = t_begin + jb;
    const int64_t count = first < t_end ? (t_end - first + bpx - 1) / bpx : 0;
    if (count == 0) return;

    // the zero slot of both buffers, and the bias
    if (tid < 4) *(uint4 *)(buf0 + WIN_CAP * W32_ROW + tid * 16) = make_uint4(0, 0, 0, 0);
    else if (tid < 8) *(uint4 *)(buf1 + WIN_CAP * W32_ROW + (tid - 4) * 16) = make_uint4(0, 0, 0, 0);
    if (tid >= 64 && tid < 96) s_bias[tid - 64] = bias ? bias[tid - 64] : 0.f;

    // weights of this wave's taps: lane holds output channel `col`, input
    // channels 16h + 8kh .. +7 (the last slot of the second half is unused)
    uint4 wf[14][2];
#pragma unroll
    for (int j = 0; j < 14; ++j) {
        const int k = 14 * th + j < 27 ? 14 * th + j : 26;
        const int kk = flip ? 26 - k : k;
#pragma unroll
        for (int h = 0; h < 2; ++h)
            wf[j][h] = *(const uint4 *)(weight + ((int64_t)col * 27 + kk) * 32 + 16 * h + 8 * kh);
    }

    auto tile_at = [&](int64_t i) { return first + i * bpx; };
    auto plan_load = [&](int64_t i) { return i < count ? plan[tile_at(i) * PLAN_INTS + (lane & 31)] : 0; };

    // prologue: plans of tiles 0, 1, 2; copies of tile 0; row numbers of tile 1
    int pv0 = plan_load(0), pv1 = plan_load(1), pv2 = plan_load(2);
    int32_t rows[W32_CHUNKS], rid[4 * W32_CHUNKS];
    {
        const W32Ranges g0 = w32_ranges(pv0);
#pragma unroll
        for (int c = 0; c < W32_CHUNKS; ++c) rows[c] = w32_row_of(perm, n, g0, 64 * (wave + W32_WAVES * c) + lane);
        w32_expand(rows, rid, lane);
#pragma unroll
        for (int it = 0; it < 4 * W32_CHUNKS; ++it) w32_copy_rows(buf0, frs, n, g0.R, rid[it], it, wave, lane, lchunk);
        w32_copy_table(buf0, nbr_sp, perm, n, tile_at(0), wave, lane);
        if (count > 1) {
            const W32Ranges g1 = w32_ranges(pv1);
#pragma unroll
            for (int c = 0; c < W32_CHUNKS; ++c) rows[c] = w32_row_of(perm, n, g1, 64 * (wave + W32_WAVES * c) + lane);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // the finished outputs of the previous tile, stored during the next one
    uint16_t *pend_out = nullptr;
    uint32_t pend[8];

    // one tile; ODD selects the buffers at compile time (the loop is unrolled by two)
    auto step = [&](auto odd, int64_t i) {
        char *cur = decltype(odd)::value ? buf1 : buf0;
        char *nxt = decltype(odd)::value ? buf0 : buf1;
        const int64_t tile = tile_at(i);
        const int R0 = plan_get(pv0, 0), R1 = plan_get(pv1, 0);
        int delta[9];
#pragma unroll
        for (int d = 0; d < 9; ++d) delta[d] = plan_get(pv0, 20 + d);
        const bool more1 = i + 1 < count, more2 = i + 2 < count;
        w32_expand(rows, rid, lane);  // row numbers of tile i+1, for its copies
        // The plan of tile i+3 and the row numbers of tile i+2, first used in the next
        // tiles, issued here in code both tap halves share: issued inside the halves they
        // were merged by register copies after them, and with copies into LDS in flight
        // a copy waits for every load outstanding.
        const int pv3 = plan_load(i + 3);
        if (more2) {
            const W32Ranges g2 = w32_ranges(pv2);
#pragma unroll
            for (int c = 0; c < W32_CHUNKS; ++c) rows[c] = w32_row_of(perm, n, g2, 64 * (wave + W32_WAVES * c) + lane);
        }

        // side work, one item per tap: 0 the table block of tile i+1 (first: it comes
        // from HBM, read once), 1-8 its row copies, 9 the stores of tile i-1
        auto side = [&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if constexpr (j == 0) {
                if (more1) w32_copy_table(nxt, nbr_sp, perm, n, tile_at(i + 1), wave, lane);
            } else if constexpr (j <= 8) {
                if (more1) w32_copy_rows(nxt, frs, n, R1, rid[j - 1], j - 1, wave, lane, lchunk);
            } else if constexpr (j == 9) {
                if (pend_out) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) *(uint2 *)(pend_out + 8 * g) = make_uint2(pend[2 * g], pend[2 * g + 1]);
                }
            }
        };

        // this wave's taps for its 32 voxels
        const int64_t s = tile * WIN_TILE + cb * 32 + col;
        const bool valid = s < n;
        const int32_t *tbl = (const int32_t *)(cur + WIN_SLOTS * W32_ROW) + (cb * 32 + col) * NBR_INTS;
        floatx16 acc = {};
        if (R0 >= 0) {
            if (th == 0) w32_taps_lds<0, 14>(acc, cur, tbl, delta, valid, kh, wf, side);
            else w32_taps_lds<14, 13>(acc, cur, tbl, delta, valid, kh, wf, side);
        } else {
            // neighbourhood too wide for the buffer: gather the rows from global memory
            if (th == 0) w32_taps_global<0, 14>(acc, feats, perm, n, tbl, valid, kh, wf, side);
            else w32_taps_global<14, 13>(acc, feats, perm, n, tbl, valid, kh, wf, side);
        }
        // combine the two tap halves through LDS
        float4 *red = s_red + cb * 256 + lane;
        if (th == 1) {  // the second tap half also adds the bias (once per output)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 bv = *(const float4 *)(s_bias + 8 * g + 4 * kh);
                red[64 * g] = make_float4(acc[4 * g] + bv.x, acc[4 * g + 1] + bv.y, acc[4 * g + 2] + bv.z,
                                          acc[4 * g + 3] + bv.w);
            }
        }
        lds_barrier();
        pend_out = nullptr;
        if (th == 0 && valid) {
            // this lane holds output channels 8g + 4kh .. +3 of its voxel, g = 0..3
            pend_out = out + (int64_t)((const int32_t *)(cur + W32_PERM))[cb * 32 + col] * 32 + 4 * kh;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 p = red[64 * g];
                const floatx2 lo = {acc[4 * g] + p.x, acc[4 * g + 1] + p.y};
                const floatx2 hi = {acc[4 * g + 2] + p.z, acc[4 * g + 3] + p.w};
                pend[2 * g] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2_t));
                pend[2 * g + 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2_t));
            }
        }
        pv0 = pv1;
        pv1 = pv2;
        pv2 = pv3;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    for (int64_t i = 0; i < count; i += 2) {
        step(std::integral_constant<int, 0>{}, i);
        if (i + 1 < count) step(std::integral_constant<int, 1>{}, i + 1);
    }
    if (pend_out) {
#pragma unroll
        for (int g = 0; g < 4; ++g) *(uint2 *)(pend_out + 8 * g) = make_uint2(pend[2 * g], pend[2 * g + 1]);
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

// Staging plan of a rulebook (part of the map build): PLAN_INTS per tile.
int64_t win_plan_ints(int64_t n) { return (n + WIN_TILE - 1) / WIN_TILE * PLAN_INTS; }

int win_plan_build(submconv_rulebook *rb, const uint32_t *blk_taps, int64_t nblk, DevStatus *st, hipStream_t s)
{
    const int64_t ntiles = (rb->n + WIN_TILE - 1) / WIN_TILE;
    if (ntiles == 0) return SUBMCONV_OK;
    // 16 lanes per tile, 16 tiles per block
    hipLaunchKernelGGL(k_win_plan, dim3((unsigned)((ntiles + PLAN_TILES - 1) / PLAN_TILES)), dim3(PLAN_THREADS), 0, s,
                       rb->gwin, rb->ngroups, ntiles, WIN_CAP, rb->plan, blk_taps, nblk, st);
    SC_LAUNCHED("win_plan");
    return SUBMCONV_OK;
}

static int device_cus(int dev)
{
    static int cached[64] = {};
    if (dev >= 0 && dev < 64 && cached[dev]) return cached[dev];
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (dev >= 0 && dev < 64) cached[dev] = cus;
    return cus;
}

bool window_supported(int cin, int cout, int dtype, int64_t n)
{
    // feature rows are addressed by 32-bit byte offsets (a buffer resource)
    return dtype == SUBMCONV_BF16 && cin == 32 && cout == 32 && n * W32_ROW <= INT32_MAX;
}

int launch_window(const void *feats, const void *w, const float *bias, const submconv_rulebook *rb,
                  void *out, int cin, int cout, int dtype, int flip, hipStream_t s)
{
    if (!window_supported(cin, cout, dtype, rb->n))
        return fail(SUBMCONV_E_UNSUPPORTED, "window kernel: bf16 with Cin = Cout = 32 and N * 64 <= 2^31 - 1 only");
    const int64_t ntiles = (rb->n + WIN_TILE - 1) / WIN_TILE;
    int blocks = device_cus(rb->device) & ~7;
    if (blocks < 8) blocks = 8;
    hipLaunchKernelGGL(k_conv_win32, dim3((unsigned)blocks), dim3(W32_WAVES * 64), 0, s, (const uint16_t *)feats,
                       (const uint16_t *)w, bias, rb->nbr_sp, rb->perm, rb->plan, (uint16_t *)out, rb->n,
                       ntiles, flip);
    SC_LAUNCHED("conv_win32");
    return SUBMCONV_OK;
}

}  // namespace sc
