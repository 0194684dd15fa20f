// Persistent matrix-core forward kernel for bf16 at 64 and 128 channels.
//
// The convolution (lato.2_mrp_mlx working notes, "Key facts" and commit
// summary): out[i, o] = bias[o] + sum_k sum_c W[o, k', c] * feats[nbr[i, k], c],
// k' = k or 26 - k (mirrored kernel), weights KRSC [Cout, 27, Cin].
//
// Implicit GEMM, transposed (out^T = W_k . F_k^T) on v_mfma_f32_16x16x32_bf16:
// the A operand is a 16-output-channel x 32-input-channel weight fragment, the
// B operand 32 input channels x 16 voxels of gathered neighbour rows.  With 16
// voxels per operand, four lanes read 64 contiguous bytes of each row, so a
// gather instruction touches half as many cache lines as with 32-voxel operands.
//
// One block per CU, 8 waves (two per SIMD).  Each block owns a contiguous run of
// 16-voxel columns (runs are split per XCD first) and walks it in rounds.  In a
// full round each wave owns CWF columns x all Cout in accumulators; the last,
// partial round splits the output tiles among the waves instead, so that a
// block's work is within a quarter column of its share.  Per round the 27 taps
// are walked with:
//   * weight tap k+1 loaded into registers at the start of tap k and written into
//     the other of two LDS buffers at its end.  Each wave reads whole rows; rows are
//     stored with a 16-byte-chunk XOR swizzle so that operand reads spread over the
//     banks.  These are ordinary loads, not direct-to-LDS copies: while such a copy
//     is in flight the compiler stops counting loads in order and waits for all of
//     them before any register operand is used;
//   * the round's block of the neighbour table in LDS (a direct copy issued after
//     the previous round's last tap, waited for before the first);
//   * B fragments loaded straight from global memory into registers, each
//     reloaded with tap k+1's data as soon as tap k's MFMAs have consumed it;
//   * neighbour rows resolved two taps ahead (table entry from LDS, then perm).
// Features, perm and weights are read as bounds-checked buffers: a missing
// neighbour is an offset past the end, which loads zeros.
#include <type_traits>

#include "common.h"

namespace sc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

constexpr int BIG_WAVES = 8;  // one block of 8 waves (two per SIMD) per CU

template <int CIN, int COUT, int NW>
struct BigShape {
    static constexpr int G = CIN / 32;          // K slices of 32 input channels per tap
    static constexpr int RT = COUT / 16;        // output tiles of 16 channels
    static constexpr int CWF = 16 / RT;         // 16-voxel columns per wave in a full round
    static constexpr int LOG_CWF = CWF >= 4 ? 2 : (CWF >= 2 ? 1 : 0);
    static constexpr int WAVES = NW;
    static constexpr int ROUND = WAVES * CWF;   // columns of a full round
    static constexpr int ROWCH = CIN / 8;       // 16-byte chunks per weight row
    static constexpr int WCH = COUT * ROWCH;    // chunks per weight tap
    static constexpr int WCOPY = (WCH + 64 * WAVES - 1) / (64 * WAVES);
    static constexpr int WBUF = WCOPY * 64 * WAVES;  // chunks per buffer (copies past WCH land in padding)
    static constexpr int AHEAD = 2;                // weight fragments read ahead of their MFMAs
    static constexpr int TCH = ROUND * 16 * NBR_INTS / 4;  // table chunks of a full round
    static constexpr int TCOPY = (TCH + 64 * WAVES - 1) / (64 * WAVES);
    static_assert(CIN % 32 == 0 && COUT % 16 == 0 && 16 % RT == 0, "tile shape");
    static_assert(CWF * RT <= 16 && CWF * G <= 8, "register budget: 64 accumulators, 32 B-operand VGPRs");
};

// Work split of one round: each wave takes CW columns x RW output tiles; PARTS
// waves share a column group; CAP columns fit in one round.
template <class S, int M>
struct BigMode {
    static constexpr int CW = (S::CWF >> M) > 0 ? (S::CWF >> M) : 1;
    static constexpr int RW = M > S::LOG_CWF ? (S::RT >> (M - S::LOG_CWF)) : S::RT;
    static constexpr int PARTS = S::RT / RW;
    static constexpr int CAP = S::WAVES / PARTS * CW;
    static_assert(RW >= 1 && S::WAVES % PARTS == 0, "mode shape");
};

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// f(integral_constant<int, I>), ..., f(integral_constant<int, N - 1>)
template <int I, int N, typename F>
__device__ __forceinline__ void big_unroll(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        big_unroll<I + 1, N>(f);
    }
}

__device__ __forceinline__ void big_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int CIN, int COUT, int NW>
struct BigCtx {
    using S = BigShape<CIN, COUT, NW>;
    const uint16_t *feats;
    const uint16_t *w;
    const float *bias;
    const int32_t *nbr_sp;
    const int32_t *perm;
    uint16_t *out;
    int64_t n;
    int flip;
    uint4 *sW0, *sW1, *sT;
    int wave, lane, s16, h;
    int32_t wofs[S::WCOPY];  // byte offset of each weight chunk this lane copies, tap 0
    int32_t aoff[S::G];      // per-lane chunk offset of each K slice's A fragment
    int64_t tlast;           // last 16-byte chunk that starts inside the table
    __amdgpu_buffer_rsrc_t rf, rp, rw;  // feats, perm and weights as bounds-checked buffers

    // weight tap k -> registers -> buf (row-major, chunk j of row o at o * ROWCH + (j ^ (o % ROWCH))).
    // Ordinary loads, not direct-to-LDS copies: with a direct copy in flight the compiler
    // stops counting loads in order and waits for every load before using any register
    // operand.
    __device__ __forceinline__ void load_w(int k, uint4 (&wr)[S::WCOPY]) const
    {
        const int32_t kofs = (flip ? 26 - k : k) * (CIN * 2);
#pragma unroll
        for (int c = 0; c < S::WCOPY; ++c)
            wr[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, wofs[c], kofs, 0));
    }
    __device__ __forceinline__ void store_w(uint4 *buf, const uint4 (&wr)[S::WCOPY]) const
    {
#pragma unroll
        for (int c = 0; c < S::WCOPY; ++c) buf[(wave + S::WAVES * c) * 64 + lane] = wr[c];
    }
    // table rows of columns [col, col + ROUND) -> sT
    __device__ __forceinline__ void stage_t(int64_t col) const
    {
        const int64_t base = col * 16 * NBR_INTS / 4;
#pragma unroll
        for (int c = 0; c < S::TCOPY; ++c) {
            int64_t q = base + (wave + S::WAVES * c) * 64 + lane;
            q = q < tlast ? q : tlast;
            __builtin_amdgcn_global_load_lds((gbl_void *)(nbr_sp + 4 * q), (lds_void *)&sT[(wave + S::WAVES * c) * 64],
                                             16, 0, 0);
        }
    }

    template <int M>
    __device__ __forceinline__ void round(int64_t col, int ncols, int64_t col_next) const
    {
        using D = BigMode<S, M>;
        constexpr int CW = D::CW, RW = D::RW, G = S::G;
        const int cg = wave / D::PARTS, r0 = (wave - cg * D::PARTS) * RW;
        const int32_t *tbl = (const int32_t *)sT;

        // Gathers use the quad layout (lane l reads 16 bytes of voxel l/4's row: four
        // consecutive lanes cover 64 contiguous bytes, half the cache-line lookups of the
        // operand layout); each fragment is then moved into the operand layout (lane l:
        // voxel l%16, chunk l/16) by four ds_bpermute.  gv* is the gathering voxel of this
        // lane, ov* the voxel whose outputs this lane holds.
        int gvloc[CW];
        bool gvok[CW], ovok[CW];
        int64_t ovrow[CW];
#pragma unroll
        for (int c = 0; c < CW; ++c) {
            const int colr = cg * CW + c;
            gvloc[c] = colr * 16 + (lane >> 2);
            gvok[c] = colr < ncols && col * 16 + gvloc[c] < n;
            const int64_t ov = col * 16 + colr * 16 + s16;
            ovok[c] = colr < ncols && ov < n;
            ovrow[c] = ovok[c] ? ov : 0;
        }
        uint32_t gmask[CW];  // presence bits of each column's voxel, read once per round
#pragma unroll
        for (int c = 0; c < CW; ++c) gmask[c] = 0;
        auto entry = [&](int k, int c) -> int32_t {
            const int d = k / 3, j = k - 3 * d;
            const uint32_t m = (gmask[c] >> (3 * d)) & 7u;
            const int32_t e = ((m >> j) & 1u) ? tbl[gvloc[c] * NBR_INTS + d] + (int32_t)__popc(m & ((1u << j) - 1u)) : -1;
            return gvok[c] ? e : -1;
        };
        // perm entry of a sorted position (the buffer load returns 0 for e = -1), and the
        // byte offset of this lane's part of that row in feats, or an offset past the end
        // for a missing neighbour (the buffer load of the row then returns zeros).  The
        // offset is formed in the tap after the perm load was issued, so its wait covers
        // that load alone, not the operand loads issued after it.
        auto perm_of = [&](int32_t e) -> int32_t { return __builtin_amdgcn_raw_buffer_load_b32(rp, e * 4, 0, 0); };
        auto offset_of = [&](int32_t r, int32_t e) -> uint32_t {
            const uint32_t miss = (uint32_t)e < (uint64_t)n ? 0u : 0x80000000u;
            return ((uint32_t)r * (CIN * 2) + 16 * (lane & 3)) | miss;
        };
        auto fload = [&](uint32_t off, int g) -> uint4 {
            return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rf, off + 64 * g, 0, 0));
        };
        const int tsrc = 4 * (4 * s16 + h);  // operand lane l takes quad lane 4 (l % 16) + l / 16
        auto tr = [&](const uint4 v) -> uint4 {
            return uint4{(uint32_t)__builtin_amdgcn_ds_bpermute(tsrc, (int)v.x),
                         (uint32_t)__builtin_amdgcn_ds_bpermute(tsrc, (int)v.y),
                         (uint32_t)__builtin_amdgcn_ds_bpermute(tsrc, (int)v.z),
                         (uint32_t)__builtin_amdgcn_ds_bpermute(tsrc, (int)v.w)};
        };

        floatx4 acc[RW][CW];
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int c = 0; c < CW; ++c) acc[r][c] = floatx4{0.f, 0.f, 0.f, 0.f};

        // prologue: the table block has landed (copied before this round)
        wait_vmcnt<0>();
        big_lds_barrier();
#pragma unroll
        for (int c = 0; c < CW; ++c) gmask[c] = (uint32_t)tbl[gvloc[c] * NBR_INTS + 9];
        uint4 wr[S::WCOPY];
        load_w(0, wr);
        int32_t orow[CW], p1[CW], e1[CW], e2[CW];  // perm and entry of tap k+1, entry of tap k+2
        uint4 F[CW][G];
#pragma unroll
        for (int c = 0; c < CW; ++c) {
            orow[c] = perm[ovrow[c]];
            asm volatile("" ::"v"(orow[c]));  // loaded here, where the prologue waits anyway
            const int32_t e0 = entry(0, c);
            const uint32_t off0 = offset_of(perm_of(e0), e0);
#pragma unroll
            for (int g = 0; g < G; ++g) F[c][g] = fload(off0, g);
            e1[c] = entry(1, c);
            p1[c] = perm_of(e1[c]);
            e2[c] = entry(2, c);
        }
        store_w(sW0, wr);
        big_lds_barrier();

        auto tap = [&](auto kc) {
            constexpr int k = decltype(kc)::value;
            const uint4 *cur = ((k & 1) ? sW1 : sW0) + r0 * 16 * S::ROWCH;
            uint4 *nxt = (k & 1) ? sW0 : sW1;
            if constexpr (k + 1 < 27) load_w(k + 1, wr);
            __builtin_amdgcn_sched_barrier(0);  // the weight loads go first: they have the whole tap to land
            uint32_t off1[CW];
            int32_t p2[CW], ep2[CW];
#pragma unroll
            for (int c = 0; c < CW; ++c) {
                if constexpr (k + 1 < 27) off1[c] = offset_of(p1[c], e1[c]);
                if constexpr (k + 2 < 27) {
                    p2[c] = perm_of(e2[c]);
                    ep2[c] = e2[c];
                }
                if constexpr (k + 3 < 27) e2[c] = entry(k + 3, c);
            }
            // A fragments i = g * RW + r, read AHEAD steps before their MFMAs; B fragments
            // of slice g + 1 moved into the operand layout while slice g computes
            constexpr int NA = G * RW, AHEAD = S::AHEAD;
            uint4 a[AHEAD + 1], T[2][CW];
#pragma unroll
            for (int c = 0; c < CW; ++c) T[0][c] = tr(F[c][0]);
#pragma unroll
            for (int i = 0; i < AHEAD && i < NA; ++i) a[i] = cur[(i % RW) * 16 * S::ROWCH + aoff[i / RW]];
#pragma unroll
            for (int i = 0; i < NA; ++i) {
                const int g = i / RW, r = i % RW;
                if (i + AHEAD < NA)
                    a[(i + AHEAD) % (AHEAD + 1)] = cur[((i + AHEAD) % RW) * 16 * S::ROWCH + aoff[(i + AHEAD) / RW]];
                if (r == 0 && g + 1 < G) {
#pragma unroll
                    for (int c = 0; c < CW; ++c) T[(g + 1) & 1][c] = tr(F[c][g + 1]);
                }
#pragma unroll
                for (int c = 0; c < CW; ++c)
                    acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[i % (AHEAD + 1)]),
                                                                        __builtin_bit_cast(bf16x8_t, T[g & 1][c]),
                                                                        acc[r][c], 0, 0, 0);
                if constexpr (k + 1 < 27) {
                    if (r == RW - 1) {
#pragma unroll
                        for (int c = 0; c < CW; ++c) F[c][g] = fload(off1[c], g);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);  // bound how far weight reads are hoisted (registers)
            }
#pragma unroll
            for (int c = 0; c < CW; ++c)
                if constexpr (k + 2 < 27) {
                    p1[c] = p2[c];
                    e1[c] = ep2[c];
                }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (k + 1 < 27) store_w(nxt, wr);
            big_lds_barrier();
        };
        big_unroll<0, 27>(tap);
        // the next round's table block: every read of this one is done (barrier after tap
        // 23), and the copy overlaps the stores below instead of the next prologue's wait
        stage_t(col_next);

        // epilogue: lane holds output channels 16 (r0 + r) + 4 h .. +3 of its voxel in column c
#pragma unroll
        for (int c = 0; c < CW; ++c) {
            if (!ovok[c]) continue;
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const int o = 16 * (r0 + r) + 4 * h;
                const float4 b = bias ? *(const float4 *)(bias + o) : make_float4(0.f, 0.f, 0.f, 0.f);
                const floatx2 lo = {acc[r][c][0] + b.x, acc[r][c][1] + b.y};
                const floatx2 hi = {acc[r][c][2] + b.z, acc[r][c][3] + b.w};
                *(uint2 *)(out + (int64_t)orow[c] * COUT + o) =
                    make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2_t)),
                               __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2_t)));
            }
        }
    }
};

template <int CIN, int COUT, int NW>
__global__ __launch_bounds__(NW * 64, 1) void k_conv_big(const uint16_t *__restrict__ feats,
                                                     const uint16_t *__restrict__ w,
                                                     const float *__restrict__ bias,
                                                     const int32_t *__restrict__ nbr_sp,
                                                     const int32_t *__restrict__ perm,
                                                     uint16_t *__restrict__ out, int64_t n, int64_t ncols,
                                                     int flip)
{
    using S = BigShape<CIN, COUT, NW>;
    __shared__ uint4 sW0[S::WBUF];
    __shared__ uint4 sW1[S::WBUF];
    __shared__ uint4 sT[S::TCOPY * 64 * S::WAVES];

    // this block's columns: the XCD's contiguous share, split evenly among its blocks
    // (contiguous runs measured faster than dealing rounds in turn among an XCD's blocks)
    const int xcd = blockIdx.x & 7, bpx = gridDim.x >> 3, jb = blockIdx.x >> 3;
    const int64_t xs = ncols * xcd / 8, xe = ncols * (xcd + 1) / 8;
    const int64_t cb = xs + (xe - xs) * jb / bpx, ce = xs + (xe - xs) * (jb + 1) / bpx;
    if (cb >= ce) return;

    BigCtx<CIN, COUT, NW> x;
    x.feats = feats; x.w = w; x.bias = bias; x.nbr_sp = nbr_sp; x.perm = perm; x.out = out;
    x.n = n; x.flip = flip; x.sW0 = sW0; x.sW1 = sW1; x.sT = sT;
    const int tid = threadIdx.x;
    x.lane = tid & 63;
    x.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    x.s16 = x.lane & 15;
    x.h = x.lane >> 4;
#pragma unroll
    for (int c = 0; c < S::WCOPY; ++c) {
        const int q = ((x.wave + S::WAVES * c) * 64 + x.lane) % S::WCH;
        const int o = q / S::ROWCH, p = q % S::ROWCH;
        x.wofs[c] = 2 * (o * 27 * CIN + 8 * (p ^ (o % S::ROWCH)));
    }
    {
        const int xr = x.h ^ (x.s16 % S::ROWCH);
#pragma unroll
        for (int g = 0; g < S::G; ++g) x.aoff[g] = x.s16 * S::ROWCH + ((4 * g) ^ xr);
    }
    x.tlast = (n * NBR_INTS + 3) / 4 - 1;
    x.rf = __builtin_amdgcn_make_buffer_rsrc((void *)feats, (short)0, (int)(n * CIN * 2), 0x00020000);
    x.rp = __builtin_amdgcn_make_buffer_rsrc((void *)perm, (short)0, (int)(n * 4), 0x00020000);
    x.rw = __builtin_amdgcn_make_buffer_rsrc((void *)w, (short)0, 27 * CIN * COUT * 2, 0x00020000);

    x.stage_t(cb);
    for (int64_t col = cb; col < ce; col += S::ROUND) {
        const int nc = (int)(ce - col < S::ROUND ? ce - col : S::ROUND);
        const int64_t nxt = col + S::ROUND < ce ? col + S::ROUND : col;
        if (nc > BigMode<S, 1>::CAP)
            x.template round<0>(col, nc, nxt);
        else if (nc > BigMode<S, 2>::CAP)
            x.template round<1>(col, nc, nxt);
        else if (nc > BigMode<S, 3>::CAP)
            x.template round<2>(col, nc, nxt);
        else
            x.template round<3>(col, nc, nxt);
    }
}

static int big_device_cus(int dev)
{
    static int cached[64] = {};
    if (dev >= 0 && dev < 64 && cached[dev]) return cached[dev];
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (dev >= 0 && dev < 64) cached[dev] = cus;
    return cus;
}

template <int CIN, int COUT, int NW>
static int launch_big_t(const void *f, const void *w, const float *b, const submconv_rulebook *rb, void *o, int flip,
                        hipStream_t s)
{
    using S = BigShape<CIN, COUT, NW>;
    const int64_t ncols = (rb->n + 15) / 16;
    int64_t blocks = big_device_cus(rb->device) & ~7;
    if (blocks < 8) blocks = 8;
    if (blocks > ((ncols + 7) & ~int64_t(7))) blocks = (ncols + 7) & ~int64_t(7);
    hipLaunchKernelGGL((k_conv_big<CIN, COUT, NW>), dim3((unsigned)blocks), dim3(S::WAVES * 64), 0, s,
                       (const uint16_t *)f, (const uint16_t *)w, b, rb->nbr_sp, rb->perm, (uint16_t *)o, rb->n,
                       ncols, flip);
    SC_LAUNCHED("conv_big");
    return SUBMCONV_OK;
}

// Features are addressed through a buffer resource with 32-bit byte offsets.
bool big_supported(int cin, int cout, int dtype, int64_t n)
{
    return dtype == SUBMCONV_BF16 && ((cin == 128 && cout == 128) || (cin == 64 && cout == 64)) &&
           n * cin * 2 <= INT32_MAX;
}

int launch_big(const void *feats, const void *w, const float *bias, const submconv_rulebook *rb, void *out,
               int cin, int cout, int dtype, int flip, hipStream_t s)
{
    if (!big_supported(cin, cout, dtype, rb->n))
        return fail(SUBMCONV_E_UNSUPPORTED,
                    "persistent kernel: bf16 with 64->64 or 128->128 channels and at most 2^31 feature bytes");
    if (cin == 128) return launch_big_t<128, 128, BIG_WAVES>(feats, w, bias, rb, out, flip, s);
    return launch_big_t<64, 64, BIG_WAVES>(feats, w, bias, rb, out, flip, s);
}

}  // namespace sc
