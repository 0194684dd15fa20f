// Persistent matrix-core forward kernel for bf16 at 64 and 128 channels.
//
// The convolution (lato.2_mrp_mlx working notes, "Key facts" and commit
// summary): out[i, o] = bias[o] + sum_k sum_c W[o, k', c] * feats[nbr[i, k], c],
// k' = k or 26 - k (mirrored kernel), weights KRSC [Cout, 27, Cin].
//
// Implicit GEMM, transposed (out^T = W_k . F_k^T) on v_mfma_f32_32x32x16_bf16:
// the A operand is a 32-output-channel x 16-input-channel weight fragment, the
// B operand 16 input channels x 32 voxels of gathered neighbour rows.
//
// One block per CU, 8 waves (two per SIMD), looping over units of sorted voxels
// (XCD-contiguous runs).  Per unit, each wave owns VT columns of 32 voxels x all
// Cout in AGPR accumulators and walks the 27 taps:
//   * weight tap k+1 is copied into the other of two LDS buffers (direct loads)
//     while tap k computes; the two buffers are two objects so the compiler
//     does not make tap k's reads wait for that copy;
//   * the B fragments are loaded straight from global memory into registers; a
//     fragment is reloaded with tap k+1's data as soon as tap k's MFMAs have
//     consumed it, so one register set serves as both operand and prefetch;
//   * neighbour rows are resolved two taps ahead (table entry, then perm).
// Every load is issued unconditionally (a missing neighbour reads a zero row),
// so the number of loads a wave issues after a weight copy is fixed; each tap
// ends by waiting until that copy has landed (vmcnt) and an LDS-only barrier,
// leaving the next tap's operand loads in flight.
#include <type_traits>

#include "common.h"

namespace sc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

__device__ uint4 g_big_zero[16] = {};  // a zero feature row (up to 128 bf16 channels)

template <int CIN, int COUT>
struct BigShape {
    static constexpr int G = CIN / 16;             // K slices of 16 input channels
    static constexpr int RT = COUT / 32;           // output row tiles of 32 channels
    static constexpr int VT = 4 / RT > 0 ? 4 / RT : 1;  // 32-voxel columns per wave
    static constexpr int NFRAG = RT * G;           // weight fragments per tap (1 KB each)
    static constexpr int WAVES = 8;
    static constexpr int UNIT = WAVES * VT * 32;   // voxels per unit
    static constexpr int WCOPY = NFRAG / WAVES;    // weight copies per wave per tap
    static_assert(NFRAG % WAVES == 0, "weight copies split evenly over the waves");
    static_assert(VT * G <= 8 && RT * VT <= 4, "register budget: 32 B-operand VGPRs, 64 accumulators");
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

template <int CIN, int COUT>
__global__ __launch_bounds__(512, 1) void k_conv_big(const uint16_t *__restrict__ feats,
                                                     const uint16_t *__restrict__ w,
                                                     const float *__restrict__ bias,
                                                     const int32_t *__restrict__ nbr_sp,
                                                     const int32_t *__restrict__ perm,
                                                     uint16_t *__restrict__ out, int64_t n,
                                                     int64_t nunits, int flip)
{
    using S = BigShape<CIN, COUT>;
    constexpr int G = S::G, RT = S::RT, VT = S::VT, NFRAG = S::NFRAG;
    __shared__ uint4 sW0[NFRAG * 64];
    __shared__ uint4 sW1[NFRAG * 64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, l32 = lane & 31;

    // units of this block: the XCD's contiguous run, dealt round-robin to its blocks
    const int xcd = blockIdx.x & 7, bpx = gridDim.x >> 3, jb = blockIdx.x >> 3;
    const int64_t u_begin = nunits * xcd / 8, u_end = nunits * (xcd + 1) / 8;

    // weight tap k -> LDS: fragment f = r G + g, lane l holds W[32 r + l%32][k'][16 g + 8 (l/32) .. +7].
    // The per-lane part of each copy's source offset is formed once; the tap part is
    // made opaque at each use, or the compiler hoists the offsets of all 27 taps and
    // holds them in registers for the whole kernel.
    int32_t wofs[S::WCOPY];
#pragma unroll
    for (int c = 0; c < S::WCOPY; ++c) {
        const int f = wave + S::WAVES * c;
        const int r = f / G, g = f - r * G;
        wofs[c] = (32 * r + l32) * 27 * CIN + 16 * g + 8 * half;
    }
    auto stage_w = [&](int k, uint4 *buf) {
        int32_t kofs = (flip ? 26 - k : k) * CIN;
        asm volatile("" : "+s"(kofs));
#pragma unroll
        for (int c = 0; c < S::WCOPY; ++c) {
            const int f = wave + S::WAVES * c;
            __builtin_amdgcn_global_load_lds((gbl_void *)(w + (uint32_t)(wofs[c] + kofs)), (lds_void *)&buf[f * 64], 16, 0, 0);
        }
    };

    for (int64_t u = u_begin + jb; u < u_end; u += bpx) {
        const int64_t vbase = (u * S::WAVES + wave) * (VT * 32);
        int64_t vrow[VT];  // clamped voxel index of each column (always a valid address)
        bool vok[VT];
#pragma unroll
        for (int t = 0; t < VT; ++t) {
            const int64_t v = vbase + 32 * t + l32;
            vok[t] = v < n;
            vrow[t] = vok[t] ? v : n - 1;
        }
        // table entry of tap k (sorted position or -1), row of a sorted position (or -1)
        auto entry = [&](int k, int t) -> int32_t {
            const int32_t e = nbr_sp[vrow[t] * 27 + k];
            return vok[t] ? e : -1;
        };
        auto row_of = [&](int32_t e) -> int32_t {
            const int32_t r = perm[(uint32_t)e < (uint64_t)n ? e : 0];
            return (uint32_t)e < (uint64_t)n ? r : -1;
        };
        auto fptr = [&](int32_t row, int g) -> const uint4 * {
            return (uint32_t)row < (uint64_t)n ? (const uint4 *)(feats + (int64_t)row * CIN + 16 * g + 8 * half)
                                               : &g_big_zero[2 * g + half];
        };

        floatx16 acc[RT][VT];
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int t = 0; t < VT; ++t)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[r][t][q] = 0.f;

        uint4 F[VT][G];
        int32_t row1[VT], e2[VT];
        // prologue: weights of tap 0, operands of tap 0, rows of tap 1, entries of tap 2
        stage_w(0, sW0);
        {
            int32_t row0[VT];
#pragma unroll
            for (int t = 0; t < VT; ++t) row0[t] = row_of(entry(0, t));
#pragma unroll
            for (int t = 0; t < VT; ++t)
#pragma unroll
                for (int g = 0; g < G; ++g) F[t][g] = *fptr(row0[t], g);
#pragma unroll
            for (int t = 0; t < VT; ++t) {
                row1[t] = row_of(entry(1, t));
                e2[t] = entry(2, t);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        big_lds_barrier();

        auto tap = [&](auto kc) {
            constexpr int k = decltype(kc)::value;
            const uint4 *cur = (k & 1) ? sW1 : sW0;
            uint4 *nxt = (k & 1) ? sW0 : sW1;
            if constexpr (k + 1 < 27) stage_w(k + 1, nxt);
            __builtin_amdgcn_sched_barrier(0);  // everything below is issued after the weight copy
            int32_t row2[VT];
#pragma unroll
            for (int t = 0; t < VT; ++t) {
                if constexpr (k + 2 < 27) row2[t] = row_of(e2[t]);
                if constexpr (k + 3 < 27) e2[t] = entry(k + 3, t);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
#pragma unroll
                for (int r = 0; r < RT; ++r) {
                    const uint4 a = cur[(r * G + g) * 64 + lane];
#pragma unroll
                    for (int t = 0; t < VT; ++t)
                        acc[r][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                                            __builtin_bit_cast(bf16x8_t, F[t][g]),
                                                                            acc[r][t], 0, 0, 0);
                }
                if constexpr (k + 1 < 27) {
#pragma unroll
                    for (int t = 0; t < VT; ++t) F[t][g] = *fptr(row1[t], g);
                }
                __builtin_amdgcn_sched_barrier(0);  // bound how far weight reads are hoisted (registers)
            }
#pragma unroll
            for (int t = 0; t < VT; ++t)
                if constexpr (k + 2 < 27) row1[t] = row2[t];
            // the weight copy of tap k+1 has landed once at most the loads issued after it are pending
            constexpr int after = ((k + 2 < 27) ? VT : 0) + ((k + 3 < 27) ? VT : 0) + ((k + 1 < 27) ? VT * G : 0);
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<after>();
            big_lds_barrier();
        };
        big_unroll<0, 27>(tap);

        // epilogue: lane holds output channels 32 r + 8 q + 4 half .. +3 of voxel column t
#pragma unroll
        for (int t = 0; t < VT; ++t) {
            if (!vok[t]) continue;
            const int64_t orow = perm[vrow[t]];
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int o = 32 * r + 8 * q + 4 * half;
                    const float4 b = bias ? *(const float4 *)(bias + o) : make_float4(0.f, 0.f, 0.f, 0.f);
                    const floatx2 lo = {acc[r][t][4 * q] + b.x, acc[r][t][4 * q + 1] + b.y};
                    const floatx2 hi = {acc[r][t][4 * q + 2] + b.z, acc[r][t][4 * q + 3] + b.w};
                    *(uint2 *)(out + orow * COUT + o) =
                        make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2_t)),
                                   __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2_t)));
                }
        }
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

template <int CIN, int COUT>
static int launch_big_t(const void *f, const void *w, const float *b, const submconv_rulebook *rb, void *o, int flip,
                        hipStream_t s)
{
    using S = BigShape<CIN, COUT>;
    const int64_t nunits = (rb->n + S::UNIT - 1) / S::UNIT;
    int64_t blocks = big_device_cus(rb->device) & ~7;
    if (blocks < 8) blocks = 8;
    if (blocks > ((nunits + 7) & ~int64_t(7))) blocks = (nunits + 7) & ~int64_t(7);
    hipLaunchKernelGGL((k_conv_big<CIN, COUT>), dim3((unsigned)blocks), dim3(S::WAVES * 64), 0, s,
                       (const uint16_t *)f, (const uint16_t *)w, b, rb->nbr_sp, rb->perm, (uint16_t *)o, rb->n,
                       nunits, flip);
    SC_LAUNCHED("conv_big");
    return SUBMCONV_OK;
}

bool big_supported(int cin, int cout, int dtype)
{
    return dtype == SUBMCONV_BF16 && ((cin == 128 && cout == 128) || (cin == 64 && cout == 64));
}

int launch_big(const void *feats, const void *w, const float *bias, const submconv_rulebook *rb, void *out,
               int cin, int cout, int dtype, int flip, hipStream_t s)
{
    if (!big_supported(cin, cout, dtype))
        return fail(SUBMCONV_E_UNSUPPORTED, "persistent kernel: bf16 with 64->64 or 128->128 channels only");
    if (cin == 128) return launch_big_t<128, 128>(feats, w, bias, rb, out, flip, s);
    return launch_big_t<64, 64>(feats, w, bias, rb, out, flip, s);
}

}  // namespace sc
