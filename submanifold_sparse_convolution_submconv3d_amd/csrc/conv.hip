// Forward kernels of the submanifold 3x3x3 convolution.
//
//   out[i, o] = bias[o] + sum_k sum_c W[o, k', c] * feats[nbr[i, k], c]
//
// over the taps k with nbr[i, k] >= 0, k' = k (correlation) or 26 - k (the
// mirrored kernel), W in KRSC layout [Cout, 27, Cin] (lato.2_mrp_mlx working
// notes, "Key facts" for the layout, commit summary for the mirror flag).
// Voxels are visited in sorted order s (the rulebook's order): the output row is
// perm[s] and the row of neighbour tap k is perm[p], p its sorted position from the
// rulebook's neighbour rows (nbr_at).  For inputs that
// arrive in grid order perm is the identity; otherwise sorted order still keeps
// a block's neighbourhoods spatially compact.
// All kernels are output-stationary: a voxel's output row is accumulated in
// registers over its 27 taps and written once, so no atomics are needed (the
// output set equals the input set).  Accumulation is fp32; a bf16 output is
// one round-to-nearest-even of the fp32 sum.
//
// Kernels:
//   generic - one thread per output element, any channel counts.
//   lowc    - Cin, Cout <= 32 on vector ALUs: a group of Cout lanes per voxel,
//             each lane loads one element of the neighbour's feature row and
//             the row is spread through the group with wave shuffles; weights
//             sit in LDS, transposed to [27][Cin][Cout].
//   mfma    - implicit GEMM on the matrix cores.  Per wave: 32*VT voxels x all
//             Cout.  The product is computed transposed, out^T = W_k . F_k^T,
//             so the MFMA A operand is a weight tap (rows = output channels)
//             and B is the gathered feature rows (columns = voxels); each lane
//             then ends up holding 4 consecutive output channels of one voxel.
//             A wave skips a tap that none of its voxels has.
#include "common.h"

namespace sc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// generic
// ---------------------------------------------------------------------------

template <typename T>
__global__ __launch_bounds__(256) void k_conv_generic(const T *__restrict__ feats,
                                                      const T *__restrict__ w,
                                                      const float *__restrict__ bias,
                                                      const int32_t *__restrict__ nbr,
                                                      const int32_t *__restrict__ perm,
                                                      T *__restrict__ out, int64_t n, int cin,
                                                      int cout, int flip)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t s = idx / cout;
    const int o = (int)(idx - s * cout);
    if (s >= n) return;
    const int64_t i = perm[s];
    if ((uint64_t)i >= (uint64_t)n) return;
    float acc = 0.f;
    for (int k = 0; k < 27; ++k) {
        const int32_t p = nbr_at(nbr + s * NBR_INTS, k);
        if ((uint32_t)p >= (uint64_t)n) continue;
        const int32_t j = perm[p];
        if ((uint32_t)j >= (uint64_t)n) continue;
        const int kw = flip ? 26 - k : k;
        const T *wr = w + ((int64_t)o * 27 + kw) * cin;
        const T *fr = feats + (int64_t)j * cin;
        for (int c = 0; c < cin; ++c) acc = fmaf(Elem<T>::to_f32(wr[c]), Elem<T>::to_f32(fr[c]), acc);
    }
    if (bias) acc += bias[o];
    out[i * cout + o] = Elem<T>::from_f32(acc);
}

// ---------------------------------------------------------------------------
// lowc: Cin, Cout <= 32, powers of two
// ---------------------------------------------------------------------------

template <typename T, int CIN, int COUT>
__global__ __launch_bounds__(256) void k_conv_lowc(const T *__restrict__ feats,
                                                   const T *__restrict__ w,
                                                   const float *__restrict__ bias,
                                                   const int32_t *__restrict__ nbr,
                                                   const int32_t *__restrict__ perm,
                                                   T *__restrict__ out, int64_t n, int flip)
{
    static_assert(COUT <= 64 && (64 % COUT) == 0, "group must divide the wave");
    constexpr int VPB = 256 / COUT;                         // voxels per block pass
    constexpr int PER = (CIN + COUT - 1) / COUT;            // feature elements per lane
    constexpr int WS = COUT + 1;                            // padded row: the scatter below hits distinct banks
    __shared__ float s_w[27 * CIN * WS];                    // [27][CIN][COUT (+1)]
    // the KRSC weights [COUT][27][CIN] read in order (whole lines), scattered transposed
    for (int e = threadIdx.x; e < 27 * CIN * COUT; e += 256) {
        const int c = e % CIN, k = (e / CIN) % 27, o = e / (27 * CIN);
        s_w[(k * CIN + c) * WS + o] = Elem<T>::to_f32(w[e]);
    }
    __syncthreads();
    const int o = threadIdx.x % COUT;
    const int lane = threadIdx.x & 63;
    const int gbase = lane - (lane % COUT);                 // first lane of this voxel's group
    const float b = bias ? bias[o] : 0.f;
    const int64_t stride = (int64_t)gridDim.x * VPB;
    // Taps in groups of G: a group's table decodes, then its row numbers, then its
    // feature loads are each issued together, so a voxel costs a few memory round
    // trips instead of two per tap.
    constexpr int G = PER <= 2 ? 27 : (PER <= 8 ? 9 : 3);
    // every lane of a wave runs the same number of iterations (shuffles need all lanes)
    for (int64_t i0 = (int64_t)blockIdx.x * VPB; i0 < n; i0 += stride) {
        const int64_t s = i0 + threadIdx.x / COUT;
        // the output row and the table row are loaded together (one round trip): both
        // loads are unconditional, at a clamped position, and checked afterwards
        const int64_t sc = s < n ? s : n - 1;
        int32_t row[NBR_INTS];
#pragma unroll
        for (int q = 0; q < NBR_INTS; ++q) row[q] = nbr[sc * NBR_INTS + q];
        const int64_t i = s < n ? (int64_t)perm[sc] : -1;
        const bool live = (uint64_t)i < (uint64_t)n;
        if (!live) row[9] = 0;  // no present taps
        float acc = 0.f;
#pragma unroll
        for (int k0 = 0; k0 < 27; k0 += G) {
            int32_t j[G];
#pragma unroll
            for (int t = 0; t < G; ++t) {
                const int32_t p = nbr_at(row, k0 + t);
                j[t] = (uint32_t)p < (uint64_t)n ? perm[p] : -1;
            }
            float f[G][PER];
#pragma unroll
            for (int t = 0; t < G; ++t)
#pragma unroll
                for (int m = 0; m < PER; ++m) {
                    const int c = o + m * COUT;
                    f[t][m] = ((uint32_t)j[t] < (uint64_t)n && c < CIN)
                                  ? Elem<T>::to_f32(feats[(int64_t)j[t] * CIN + c]) : 0.f;
                }
#pragma unroll
            for (int t = 0; t < G; ++t) {
                const int k = k0 + t;
                const float *wk = s_w + (flip ? 26 - k : k) * CIN * WS + o;
#pragma unroll
                for (int c = 0; c < CIN; ++c) {
                    const float fc = __shfl(f[t][c / COUT], gbase + (c % COUT), 64);
                    acc = fmaf(wk[c * WS], fc, acc);
                }
            }
        }
        if (live) out[i * COUT + o] = Elem<T>::from_f32(acc + b);
    }
}

// ---------------------------------------------------------------------------
// mfma16: Cin = Cout = 16 on the matrix cores
//
// One wave per column of 16 sorted voxels, computed transposed (out^T = W_k . F_k^T:
// rows = output channels, columns = voxels).  Lane l = 16 q + m holds weight row m
// (output channel m) and voxel m of the column, at input channels 4q .. 4q + 3; fp32
// contracts them in four v_mfma_f32_16x16x4f32 steps (step e: channel 4q + e on both
// operands), bf16 in one v_mfma_f32_16x16x16bf16_1k.  The result leaves lane l with
// output channels 4q .. 4q + 3 of voxel m.  All 27 weight taps stay in registers, and
// a column's neighbour rows are fetched through buffer resources: a missing neighbour
// is an offset past the end, which reads zeros, so no load sits behind a branch.
// ---------------------------------------------------------------------------

typedef short shortx4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Mfma16 {
    static constexpr int G = 9;                                      // taps per batch of loads
    using Frag = floatx4;                                            // 4 input channels
    static __device__ __forceinline__ Frag load(__amdgpu_buffer_rsrc_t r, uint32_t off)
    {
        return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
    static __device__ __forceinline__ void mma(floatx4 &acc, const Frag &a, const Frag &b)
    {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
    }
};
template <>
struct Mfma16<uint16_t> {
    static constexpr int G = 27;
    using Frag = shortx4;
    static __device__ __forceinline__ Frag load(__amdgpu_buffer_rsrc_t r, uint32_t off)
    {
        return __builtin_bit_cast(shortx4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    }
    static __device__ __forceinline__ void mma(floatx4 &acc, const Frag &a, const Frag &b)
    {
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
    }
};

template <typename T>
__global__ __launch_bounds__(64) void k_conv_mfma16(const T *__restrict__ feats, const T *__restrict__ w,
                                                    const float *__restrict__ bias,
                                                    const int32_t *__restrict__ nbr,
                                                    const int32_t *__restrict__ perm, T *__restrict__ out,
                                                    int64_t n, int flip)
{
    using M = Mfma16<T>;
    using Frag = typename M::Frag;
    constexpr uint32_t ROW = 16 * sizeof(T), OOB = 0x80000000u;  // bytes per feature row; past every end
    const int lane = threadIdx.x, m = lane & 15, q = lane >> 4;
    const __amdgpu_buffer_rsrc_t rf = __builtin_amdgcn_make_buffer_rsrc((void *)feats, (short)0, (int)(n * ROW), 0x00020000);
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc((void *)perm, (short)0, (int)(n * 4), 0x00020000);
    Frag wf[27];
#pragma unroll
    for (int k = 0; k < 27; ++k)
        wf[k] = *(const Frag *)(w + ((int64_t)m * 27 + (flip ? 26 - k : k)) * 16 + 4 * q);
    float bv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) bv[r] = bias ? bias[4 * q + r] : 0.f;
    const int64_t ncol = (n + 15) / 16;
    for (int64_t col = blockIdx.x; col < ncol; col += gridDim.x) {
        // the voxel's table row and its output row, loaded together at a clamped position
        const int64_t s = col * 16 + m, sc = s < n ? s : n - 1;
        int32_t row[NBR_INTS];
#pragma unroll
        for (int e = 0; e < NBR_INTS; ++e) row[e] = nbr[sc * NBR_INTS + e];
        const int64_t i = s < n ? (int64_t)perm[sc] : -1;
        const bool live = (uint64_t)i < (uint64_t)n;
        if (!live) row[9] = 0;  // no present taps
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < 27; k0 += M::G) {
            bool ok[M::G];
            int32_t j[M::G];
#pragma unroll
            for (int t = 0; t < M::G; ++t) {
                const int32_t p = nbr_at(row, k0 + t);
                ok[t] = (uint32_t)p < (uint64_t)n;
                j[t] = __builtin_amdgcn_raw_buffer_load_b32(rp, ok[t] ? (uint32_t)p * 4u : OOB, 0, 0);
            }
            Frag f[M::G];
#pragma unroll
            for (int t = 0; t < M::G; ++t)
                f[t] = M::load(rf, ok[t] ? (uint32_t)j[t] * ROW + (uint32_t)q * (ROW / 4) : OOB);
#pragma unroll
            for (int t = 0; t < M::G; ++t) M::mma(acc, wf[k0 + t], f[t]);
        }
        if (live) {
            T y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = Elem<T>::from_f32(acc[r] + bv[r]);
            if constexpr (sizeof(T) == 4) *(float4 *)(out + i * 16 + 4 * q) = *(const float4 *)y;
            else *(uint2 *)(out + i * 16 + 4 * q) = *(const uint2 *)y;
        }
    }
}

bool mfma16_supported(int cin, int cout, int dtype, int64_t n)
{
    // feature rows are addressed by 32-bit byte offsets (a buffer resource)
    return cin == 16 && cout == 16 && n * 16 * (dtype == SUBMCONV_F32 ? 4 : 2) <= INT32_MAX;
}

template <typename T>
static void launch_mfma16_t(const void *f, const void *w, const float *b, const int32_t *nbr, const int32_t *perm,
                            void *o, int64_t n, int flip, hipStream_t s)
{
    int64_t waves = (n + 15) / 16;  // one 16-voxel column per wave; up to 8 waves per CU
    if (waves > 2048) waves = 2048;
    hipLaunchKernelGGL(k_conv_mfma16<T>, dim3((unsigned)waves), dim3(64), 0, s, (const T *)f, (const T *)w, b, nbr,
                       perm, (T *)o, n, flip);
}

// ---------------------------------------------------------------------------
// mfma: implicit GEMM on the matrix cores
//
// bf16 uses v_mfma_f32_32x32x16_bf16, fp32 uses v_mfma_f32_32x32x2_f32 four
// times per 16-byte fragment.  Operand layout (both): a 1 KB fragment holds,
// in lane l, the 16 bytes of matrix row (l % 32) at 16-byte chunk 2g + l / 32
// of that row, where g is the fragment's group along Cin.  For bf16 a chunk is
// 8 channels and the 32x32x16 instruction contracts both halves at once; for
// fp32 a chunk is 4 channels and step e of the four 32x32x2 instructions takes
// element e of both lanes' chunks, so each group covers its 8 channels once.
// (The contraction order may be permuted freely as long as A and B agree.)
// D (32 x 32): lane l holds column l % 32, rows 8 (q/4) + 4 (l/32) + q % 4.
//
// Data movement of the persistent fp32 128 -> 128 kernel below (8 waves per
// block, each a 32-voxel column x all Cout in a full round):
//   * weight tap k' is copied once per block into LDS in fragment order by
//     direct global->LDS loads (no register staging), double-buffered so the
//     copy of the next tap overlaps this tap's MFMAs;
//   * the B operand (gathered feature rows) is loaded straight into registers,
//     one tap ahead of the MFMAs that use it; a missing neighbour reads the
//     zero row.
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

__device__ uint4 g_zero_row[64] = {};  // 1 KB of zeros: the row of a missing neighbour

// nbr_at with both table words read unconditionally: no branch, so a lookup can sit
// between MFMA groups without splitting their scheduling region
__device__ __forceinline__ int32_t nbr_at_flat(const int32_t *row, int k)
{
    const int d = k / 3, j = k - 3 * d;
    const uint32_t m = ((uint32_t)row[9] >> (3 * d)) & 7u;
    const int32_t first = row[d];
    // (an OR with the absent mask, not a select: a value used under a condition lets the
    // compiler move its load into a branch)
    const int32_t absent = (int32_t)((m >> j) & 1u) - 1;  // 0 present, -1 absent
    return (first + (int32_t)__popc(m & ((1u << j) - 1u))) | absent;
}

// s_waitcnt with only the LDS/scalar counter at zero (vector-memory loads may stay in flight)
#define SC_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

// Copy the neighbour-table rows of voxels [v0, v0 + nvox) into LDS (direct loads,
// 1 KB per wave instruction).  The table allocation is padded, so a 16-byte chunk
// that straddles its end stays inside it; chunks wholly past the end read zeros
// (those voxels do not exist and their entries are never used).
template <int NVOX, int NWAVES = 4>
__device__ __forceinline__ void stage_nbr(const int32_t *nbr, int64_t n, int64_t v0, char *dst,
                                          int wave, int lane)
{
    constexpr int NI = (NVOX * NBR_INTS * 4 + 1023) / 1024;
    const char *base = (const char *)(nbr + v0 * NBR_INTS);
    const int64_t left = (n - v0) * NBR_INTS * 4;  // valid bytes from base
    for (int i = wave; i < NI; i += NWAVES) {
        const int64_t off = (int64_t)i * 1024 + lane * 16;
        const void *src = off < left ? (const void *)(base + off) : (const void *)g_zero_row;
        __builtin_amdgcn_global_load_lds((gbl_void *)src, (lds_void *)(dst + i * 1024), 16, 0, 0);
    }
}

// Block index remapped so that each of the 8 XCDs (workgroup id mod 8) takes a
// contiguous run of blocks: consecutive sorted voxels share neighbours, so the
// run's gathers stay within one L2 instead of every L2 seeing the whole set.
__device__ __forceinline__ int64_t xcd_block()
{
    const int64_t g = gridDim.x, b = blockIdx.x;
    const int64_t q = g >> 3, r = g & 7, x = b & 7;
    return x * q + (x < r ? x : r) + (b >> 3);
}

template <typename T> struct Mma;
template <> struct Mma<uint16_t> {
    static __device__ __forceinline__ void step(floatx16 &acc, const uint4 &a, const uint4 &b)
    {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                      __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
    }
};
template <> struct Mma<float> {
    static __device__ __forceinline__ void step(floatx16 &acc, const uint4 &a, const uint4 &b)
    {
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
    }
};

template <typename T> struct Store4;
template <> struct Store4<uint16_t> {
    static __device__ __forceinline__ void put(uint16_t *p, float a, float b, float c, float d)
    {
        const uint32_t lo = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16);
        *(uint2 *)p = make_uint2(lo, hi);
    }
};
template <> struct Store4<float> {
    static __device__ __forceinline__ void put(float *p, float a, float b, float c, float d)
    {
        *(float4 *)p = make_float4(a, b, c, d);
    }
};

template <typename T, int CIN, int COUT, int VT>
struct MfmaShape {
    static constexpr int ES = (int)sizeof(T);
    static constexpr int EPC = 16 / ES;                // elements per 16-byte chunk
    static constexpr int G = CIN * ES / 32;            // fragment groups along Cin
    static constexpr int RT = COUT / 32;               // row tiles (output channels)
    static constexpr int NFRAG = RT * G;               // weight fragments per tap (1 KB each)
    static_assert(G >= 1 && RT >= 1, "channel counts too small for the matrix-core path");
};

// Persistent: one block of 8 waves per CU (two per SIMD, so that one wave's
// copy-issue and LDS stalls hide behind the other's MFMAs) walks 32-voxel columns
// in rounds: the blocks of an XCD take its eighth of the columns together, one
// round of 8 columns each in turn, and then split the columns left over evenly.
// In a full round each wave owns one column and all Cout; in the last, partial
// round the waves share the remaining columns and split Cout so that no SIMD
// carries more than it must.  With one block per CU, a grid of fixed-size blocks
// ran whole extra rounds on some CUs while the rest idled; with each block on its
// own contiguous run, an XCD's L2 saw 32 separate windows of rows and fetched each
// row from memory about twice as often.
constexpr int MFMA_P_WAVES = 8;

template <typename T, int CIN, int COUT, int VT>
__global__ __launch_bounds__(64 * MFMA_P_WAVES) void k_conv_mfma(const T *__restrict__ feats,
                                                                  const T *__restrict__ w,
                                                                  const float *__restrict__ bias,
                                                                  const int32_t *__restrict__ nbr,
                                                                  const int32_t *__restrict__ perm,
                                                                  T *__restrict__ out, int64_t n, int flip)
{
    using S = MfmaShape<T, CIN, COUT, VT>;
    constexpr int WV = MFMA_P_WAVES, VPB = 32 * WV;
    constexpr int G = S::G, RT = S::RT, NFRAG = S::NFRAG, EPC = S::EPC;
    constexpr int NW = NFRAG / WV;  // weight fragments each wave copies per tap
    static_assert(VT == 1 && RT % 4 == 0, "one column per wave, Cout split in quarters in a partial round");
    static_assert(CIN * (int)sizeof(T) <= 1024, "a feature row fits the zero row");
    static_assert(NFRAG % WV == 0 && NW <= G / 2 && G % 2 == 0, "the next tap's copies fit the first half of the MFMA groups");
    // two weight objects: the compiler tracks direct global-to-LDS copies per object,
    // so reading tap k's buffer does not wait for the copy of tap k+1 into the other
    // (and, through it, for every load in flight)
    __shared__ uint4 sW0[1][NFRAG * 64];
    __shared__ uint4 sW1[1][NFRAG * 64];
    __shared__ __attribute__((aligned(16))) int32_t sN[VPB * NBR_INTS + 256];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t ncols = (n + 31) / 32;
    // Columns: with a grid of whole XCDs (workgroup id mod 8), each XCD takes a
    // contiguous eighth of the columns and its blocks walk it together, full rounds
    // dealt in turn (round rd of block j: columns xs + (rd * bpx + j) * WV ..), so the
    // XCD's gathers stay within a narrow window of sorted voxels that its L2 holds;
    // the columns left over are then split evenly among the XCD's blocks.  Otherwise
    // each block takes one balanced contiguous run.
    int64_t full_base = 0, full_step = 0, c0, c1;
    int full;
    if ((gridDim.x & 7) == 0) {
        const int64_t xcd = blockIdx.x & 7, bpx = gridDim.x >> 3, jb = blockIdx.x >> 3;
        const int64_t xs = ncols * xcd / 8, xe = ncols * (xcd + 1) / 8;
        const int64_t nfull = (xe - xs) / (WV * bpx);
        full = (int)nfull;
        full_base = xs + jb * WV;
        full_step = bpx * WV;
        const int64_t rb0 = xs + nfull * WV * bpx, rt = xe - rb0;
        c0 = rb0 + rt * jb / bpx;
        c1 = rb0 + rt * (jb + 1) / bpx;
    } else {
        const int64_t blk = xcd_block();
        c0 = ncols * blk / gridDim.x;
        c1 = ncols * (blk + 1) / gridDim.x;
        full = 0;
    }
    const int m = (int)(c1 - c0);
    if (m <= 0 && full == 0) return;

    // copy weight fragment f of tap k (kernel tap k' = flip ? 26-k : k) into `dst`
    auto copy_w = [&](int k, uint4 *dst, int f) {
        const int kw = flip ? 26 - k : k;
        const int r = f / G, g = f - r * G;
        const T *src = w + ((int64_t)(32 * r + l32) * 27 + kw) * CIN + (2 * g + half) * EPC;
        __builtin_amdgcn_global_load_lds((gbl_void *)src, (lds_void *)&dst[f * 64], 16, 0, 0);
    };
    auto stage_w = [&](int k, uint4 *dst) {
#pragma unroll
        for (int i = 0; i < NW; ++i) copy_w(k, dst, wave + WV * i);
    };

    // One round over the columns col0 .. (up to 8): this wave's column `col` (its
    // voxels at sN rows (col - col0) * 32 ..), output tiles r0 .. r0 + RTW - 1.  An
    // inactive wave only copies its share of the weights and meets the barriers.
    auto round = [&](auto rtw, int64_t col0, int64_t col, int r0, bool active) {
        constexpr int RTW = decltype(rtw)::value;
        const int64_t vbase = col * 32;
        const int srow = (int)(col - col0) * 32;

        // the previous round's readers of sN and of the weight buffers are done
        __syncthreads();
        stage_w(0, sW0[0]);
        stage_nbr<VPB, WV>(nbr, n, col0 * 32, (char *)sN, wave, lane);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        if (!active) {
            for (int k = 0; k < 26; k += 2) {
                stage_w(k + 1, sW1[0]);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                stage_w(k + 2, sW0[0]);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            }
            return;
        }

        // input rows of this wave's voxels' tap-k neighbours, looked up a tap before
        // their fragments are fetched: the perm loads are unconditional and not
        // inspected here, so they overlap a tap of MFMAs instead of being waited on
        struct Look {
            int32_t r;
            bool ok;
        };
        auto lookup = [&](int k) -> Look {
            const int64_t v = vbase + l32;
            const int32_t e = nbr_at_flat(sN + (srow + l32) * NBR_INTS, k) | -(int32_t)(v >= n);
            Look L;
            L.ok = (uint32_t)e < (uint64_t)n;
            L.r = perm[L.ok ? e : 0];
            return L;
        };
        // first chunk of this lane's feature fragments for a looked-up row: the row
        // itself, or the zero row for a missing neighbour (an address choice, so every
        // fragment is one unconditional load)
        auto frag_src = [&](const Look &L) -> const T * {
            const bool real = L.ok && (uint32_t)L.r < (uint64_t)n;
            return (real ? feats + (int64_t)L.r * CIN : (const T *)g_zero_row) + half * EPC;
        };

        floatx16 acc[RTW];
#pragma unroll
        for (int r = 0; r < RTW; ++r)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[r][q] = 0.f;

        // tap k's MFMAs (weights in LDS buffer wb, features in F).  With PF the next
        // tap's copies go out piece by piece between the MFMA groups of the first half
        // of the tap: group g < G/2 brings feature fragments 2g, 2g+1 into Fn and
        // weight fragment g of this wave's share into wn (issued all at once, a wave's
        // copies stalled its issue for about a third of a tap; issued through the whole
        // tap, the last gathers were still in flight at its end).  The groups are kept
        // apart so that the copies stay spread and the registers of only one group's
        // LDS reads are live.
        auto compute = [&](auto pf, const uint4 *wb, const uint4 (&F)[G], int kn, uint4 *wn,
                           const T *fsrc, uint4 (&Fn)[G], auto &&after_first) {
            constexpr bool PF = decltype(pf)::value;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (g == 1) after_first();
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (PF) {
                    if (g < G / 2) {
                        Fn[2 * g] = *(const uint4 *)(fsrc + 4 * g * EPC);
                        Fn[2 * g + 1] = *(const uint4 *)(fsrc + (4 * g + 2) * EPC);
                    }
                    if (g < NW) copy_w(kn, wn, wave + WV * g);
                }
#pragma unroll
                for (int r = 0; r < RTW; ++r) {
                    const uint4 a = wb[((r0 + r) * G + g) * 64 + lane];
                    Mma<T>::step(acc[r], a, F[g]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        };

        uint4 F0[G], F1[G];
        {
            const T *src = frag_src(lookup(0));
#pragma unroll
            for (int g = 0; g < G; ++g) F0[g] = *(const uint4 *)(src + 2 * g * EPC);
        }
        Look Ln = lookup(1);  // the next tap's rows
        __builtin_amdgcn_s_waitcnt(0);

        // taps 0..25: copy tap k+1 (weights into the other LDS buffer, features into
        // the other register set) during tap k's MFMAs, look up tap k+2, then wait and
        // meet at a barrier.  ODD (the loop is unrolled by two) picks the weight
        // buffers at compile time.  Taps run even where no voxel of the column has the
        // neighbour (well under 1% of column-taps on surface-like sets): a branch
        // around the MFMAs made the compiler copy the accumulators on every tap.
        // (the lookup of tap k+2 follows the first MFMA group: ahead of it, its LDS and
        // perm round trips held the start of every tap)
        auto tap = [&](auto odd, int k, uint4 (&Fc)[G], uint4 (&Fn)[G]) {
            constexpr bool O = decltype(odd)::value;
            const T *fsrc = frag_src(Ln);
            compute(std::true_type{}, O ? sW1[0] : sW0[0], Fc, k + 1, O ? sW0[0] : sW1[0], fsrc, Fn,
                    [&] { Ln = lookup(k + 2 < 27 ? k + 2 : 26); });
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        };
        for (int k = 0; k < 26; k += 2) {
            tap(std::false_type{}, k, F0, F1);
            tap(std::true_type{}, k + 1, F1, F0);
        }
        // tap 26 (even: buffer 0, register set 0), nothing left to copy
        compute(std::false_type{}, sW0[0], F0, 26, sW1[0], (const T *)g_zero_row, F1, [] {});

        const int64_t v = vbase + l32;
        if (v >= n) return;
        const int64_t orow = perm[v];
        if ((uint64_t)orow >= (uint64_t)n) return;
#pragma unroll
        for (int r = 0; r < RTW; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int o = 32 * (r0 + r) + 8 * q + 4 * half;
                float4 bv = make_float4(0.f, 0.f, 0.f, 0.f);
                if (bias) bv = *(const float4 *)(bias + o);
                Store4<T>::put(out + orow * COUT + o, acc[r][4 * q] + bv.x, acc[r][4 * q + 1] + bv.y,
                               acc[r][4 * q + 2] + bv.z, acc[r][4 * q + 3] + bv.w);
            }
    };

    // waves w and w + 4 share a SIMD; each partial-round split below gives every SIMD
    // at most the quarter-tile work the columns need (rem 5..7 cost a full round)
    using Q = std::integral_constant<int, RT / 4>;
    using H = std::integral_constant<int, RT / 2>;
    using A = std::integral_constant<int, RT>;
    for (int rd = 0; rd < full; ++rd) {
        const int64_t cf = full_base + full_step * rd;
        round(A{}, cf, cf + wave, 0, true);
    }
    const int mfull = m / WV, rem = m % WV;
    for (int rd = 0; rd < mfull; ++rd)
        round(A{}, c0 + WV * rd, c0 + WV * rd + wave, 0, true);
    const int64_t ct = c0 + WV * mfull;
    if (rem == 1)  // waves 0..3 (one per SIMD): a quarter of Cout each
        round(Q{}, ct, ct, (wave & 3) * (RT / 4), wave < 4);
    else if (rem == 2)  // 4 waves per column, a quarter each
        round(Q{}, ct, ct + (wave >> 2), (wave & 3) * (RT / 4), true);
    else if (rem == 3)  // 2 waves per column, a half each (waves 6, 7 idle)
        round(H{}, ct, ct + (wave < 6 ? wave >> 1 : 0), (wave & 1) * (RT / 2), wave < 6);
    else if (rem == 4)
        round(H{}, ct, ct + (wave >> 1), (wave & 1) * (RT / 2), true);
    else if (rem > 4)
        round(A{}, ct, ct + (wave < rem ? wave : 0), 0, wave < rem);
}

// ---------------------------------------------------------------------------
// mfma, row-gathered operands (used where its LDS fits)
//
// Same MFMA fragments as above, but operands travel through LDS as whole
// rows: a direct global->LDS load moves 1 KB per wave instruction, 64 lanes
// x 16 bytes, with consecutive lanes covering consecutive 16-byte chunks of
// one row, so each gathered feature row (and each weight row) is fetched as
// whole cache lines.  Inside LDS a row's chunk c sits in slot c ^ sw(row),
// an XOR swizzle that puts the 16 rows read by 16 consecutive lanes in 16
// different bank groups, so fragment reads are free of bank conflicts.
// Missing neighbours load from a zero row.  Per wave, the next tap's rows are
// gathered into its private LDS region while the current tap's MFMAs run
// (the B fragments of the current tap having been read into registers first).
// ---------------------------------------------------------------------------

template <int RB>  // row bytes
__device__ __forceinline__ int swz(int row)
{
    constexpr int CH = RB / 16;                   // 16-byte chunks per row
    if constexpr (CH >= 16) return row & 15;
    else return (row / (16 / CH)) & (CH - 1);
}

constexpr int align1k(int b) { return (b + 1023) & ~1023; }

// OS output groups: the OS waves of a column share its gathered rows and split
// Cout, so a block covers 4/OS columns (more blocks on small sets, less MFMA work
// per wave).  A shared column region is double-buffered: one wave may gather tap
// k+1 while the other still reads tap k.
template <typename T, int CIN, int COUT, int VT, int OS = 1>
struct RowShape {
    static constexpr int ES = (int)sizeof(T);
    static constexpr int RB = CIN * ES;                // bytes per feature / weight row
    static constexpr int CH = RB / 16;                 // chunks per row
    static constexpr int RPI = 1024 / RB;              // rows per 1 KB load instruction
    static constexpr int EPC = 16 / ES;
    static constexpr int G = CH / 2;
    static constexpr int RT = COUT / 32 / OS;          // 32-output tiles per wave
    static constexpr int ROWS = VT * 32;               // gathered rows per column
    static constexpr int COLS = 4 / OS;                // columns per block
    static constexpr int FB = OS == 1 ? 1 : 2;         // row buffers per column
    static constexpr int W_TAP = COUT * RB;            // bytes of one weight tap
    static constexpr bool RESIDENT = 27 * W_TAP <= 65536;
    static constexpr int WBUF = RESIDENT ? 27 : 2;
    static constexpr int VOX_PER_BLOCK = COLS * ROWS;
    static constexpr int NBR_BYTES = VOX_PER_BLOCK * NBR_INTS * 4;
    // the kernel's objects: weights (one object of 27 taps, or two of one tap), one
    // or two row buffers, the table block; 1-KB alignment of each
    static constexpr int LDS = (RESIDENT ? align1k(27 * W_TAP) + 1024 : 2 * align1k(W_TAP)) +
                               (FB == 2 ? 2 : 1) * align1k(COLS * ROWS * RB) + (FB == 2 ? 0 : 1024) +
                               align1k(NBR_BYTES);
    static_assert(RB >= 64 && RB <= 1024 && (RB & (RB - 1)) == 0, "row size");
    static_assert(OS == 1 || OS == 2, "output groups");
    static_assert(RT >= 1 && RT * 32 * OS == COUT, "Cout split");
    static_assert((ROWS / RPI) % OS == 0, "gather instructions split evenly");
};

template <typename T, int CIN, int COUT, int VT, int OS>
__global__ __launch_bounds__(256) void k_conv_mfma_rows(const T *__restrict__ feats,
                                                        const T *__restrict__ w,
                                                        const float *__restrict__ bias,
                                                        const int32_t *__restrict__ nbr,
                                                        const int32_t *__restrict__ perm,
                                                        T *__restrict__ out, int64_t n, int flip)
{
    using S = RowShape<T, CIN, COUT, VT, OS>;
    constexpr int RB = S::RB, CH = S::CH, RPI = S::RPI, EPC = S::EPC, G = S::G, RT = S::RT;
    constexpr int ROWS = S::ROWS, COLS = S::COLS, FB = S::FB;
    // One object per region and buffer: the compiler tracks direct global-to-LDS
    // copies per object, so reading one buffer does not wait for copies into another
    // (within one object every LDS read waited for every copy in flight).
    __shared__ __attribute__((aligned(1024))) char sW0[S::RESIDENT ? 27 * S::W_TAP : S::W_TAP];
    __shared__ __attribute__((aligned(1024))) char sW1[S::RESIDENT ? 16 : S::W_TAP];
    __shared__ __attribute__((aligned(1024))) char sF0[COLS * ROWS * RB];
    __shared__ __attribute__((aligned(1024))) char sF1[FB == 2 ? COLS * ROWS * RB : 16];
    __shared__ __attribute__((aligned(1024))) char sNb[S::NBR_BYTES];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int colw = wave / OS, og = wave % OS;                 // column, output group
    const int32_t *sN = (const int32_t *)sNb;                   // [block voxels][NBR_INTS]
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t blk = xcd_block();
    const int64_t vbase = (blk * COLS + colw) * ROWS;

    // weight tap k -> `dst` (one tap: [COUT rows][RB]), whole rows, swizzled
    auto stage_w = [&](int k, char *dst) {
        const int kw = flip ? 26 - k : k;
        constexpr int NI = COUT / RPI;                          // 1 KB instructions per tap
        for (int i = wave; i < NI; i += 4) {
            const int o = i * RPI + lane / CH;
            const int c = (lane % CH) ^ swz<RB>(o);
            const T *src = w + ((int64_t)o * 27 + kw) * CIN + c * EPC;
            __builtin_amdgcn_global_load_lds((gbl_void *)src, (lds_void *)(dst + i * 1024), 16, 0, 0);
        }
    };
    // input row of the tap-k neighbour of the column's voxel `lane` (lanes < ROWS):
    // looked up one tap before its gather, so the load overlaps a tap of MFMAs.  The
    // load is unconditional and its value is not inspected here (either would make
    // the compiler wait for it at once); the gather applies the checks.
    struct Look {
        int32_t r;
        bool ok;
    };
    auto lookup = [&](int k) -> Look {
        // branch-free (lanes past the column read its last row and are dropped), so that
        // it can sit between MFMA groups without splitting them
        const int32_t e = nbr_at_flat(sN + (colw * ROWS + (lane < ROWS ? lane : ROWS - 1)) * NBR_INTS, k) |
                          -(int32_t)(lane >= ROWS || vbase + lane >= n);
        const bool ok = (uint32_t)e < (uint64_t)n;
        return Look{perm[ok ? e : 0], ok};
    };
    // row to gather for a looked-up entry, or -1 (the zero row)
    auto row_of = [&](const Look &L) -> int32_t { return L.ok && (uint32_t)L.r < (uint64_t)n ? L.r : -1; };
    // copy q of the column's neighbour rows into its region of `fbuf`: the OS waves of
    // the column each issue every OS-th 1 KB copy; a missing neighbour copies the zero
    // row (an address choice, so the copy is unconditional)
    constexpr int NGP = (ROWS / RPI) / OS;  // row copies per wave and tap
    auto spread_rows = [&](int32_t j, int32_t (&jr)[NGP]) {  // row of each copy's lane
#pragma unroll
        for (int q = 0; q < NGP; ++q) jr[q] = __shfl(j, (og + OS * q) * RPI + lane / CH, 64);
    };
    auto gather_piece = [&](const int32_t (&jrs)[NGP], char *fbuf, int q) {
        const int i = og + OS * q;
        const int row = i * RPI + lane / CH;
        const int jr = jrs[q];
        const int c = (lane % CH) ^ swz<RB>(row);
        const void *src = jr >= 0 ? (const void *)(feats + (int64_t)jr * CIN + c * EPC)
                                  : (const void *)((const char *)g_zero_row + c * 16);
        __builtin_amdgcn_global_load_lds((gbl_void *)src, (lds_void *)(fbuf + colw * ROWS * RB + i * 1024), 16, 0, 0);
    };
    // weight copy p of this wave for tap k (instruction wave + 4p of the tap; a wave
    // with fewer repeats its last one, which writes the same bytes again)
    constexpr int NI_W = COUT / RPI;
    constexpr int NWP = S::RESIDENT ? 0 : (NI_W + 3) / 4;
    auto copy_w_piece = [&](int k, char *dst, int p) {
        const int kw = flip ? 26 - k : k;
        const int i = wave + 4 * p < NI_W ? wave + 4 * p : NI_W - 1;
        const int o = i * RPI + lane / CH;
        const int c = (lane % CH) ^ swz<RB>(o);
        const T *src = w + ((int64_t)o * 27 + kw) * CIN + c * EPC;
        __builtin_amdgcn_global_load_lds((gbl_void *)src, (lds_void *)(dst + i * 1024), 16, 0, 0);
    };

    floatx16 acc[RT][VT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int t = 0; t < VT; ++t)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[r][t][q] = 0.f;

    if constexpr (S::RESIDENT) {
        for (int k = 0; k < 27; ++k) stage_w(k, sW0 + k * S::W_TAP);
    } else {
        stage_w(0, sW0);
    }
    stage_nbr<S::VOX_PER_BLOCK>(nbr, n, blk * S::VOX_PER_BLOCK, sNb, wave, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    {
        int32_t jr0[NGP];
        spread_rows(row_of(lookup(0)), jr0);
#pragma unroll
        for (int q = 0; q < NGP; ++q) gather_piece(jr0, sF0, q);
    }
    Look jn = lookup(1);  // the next tap's rows

    // Tap k; ODD picks the buffers at compile time (the tap loop is unrolled by two):
    // weights and rows of tap k are read from one buffer while tap k+1 fills the
    // other.  With PF (taps 0..25) the next tap's copies are issued a few at a time
    // between the MFMA groups of the first half of the tap: issued together at its
    // start they held the wave's issue for a large part of it.  Every tap runs its MFMAs (a branch around
    // them made the compiler copy the accumulators each tap).
    auto step = [&](auto odd, auto pf, int k) {
        constexpr bool O = decltype(odd)::value, PF = decltype(pf)::value;
        char *wnxt = O ? sW0 : sW1;
        char *fcur = (FB == 2 && O) ? sF1 : sF0;
        char *fnxt = (FB == 2 && !O) ? sF1 : sF0;
        const char *wb = S::RESIDENT ? sW0 + k * S::W_TAP : (O ? sW1 : sW0);
        __builtin_amdgcn_s_waitcnt(0);   // this wave's loads into LDS have landed
        __syncthreads();                 // ... and everyone's; the other buffers are free
        uint4 F[VT][G];
        {
            const char *src = fcur + colw * ROWS * RB;
#pragma unroll
            for (int t = 0; t < VT; ++t)
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int row = 32 * t + l32;
                    F[t][g] = *(const uint4 *)(src + row * RB + (((2 * g + half) ^ swz<RB>(row)) << 4));
                }
        }
        // With one row buffer the fragments must be in registers before this wave
        // refills its region; with two, the next gather goes to the other buffer, which
        // every wave of the column finished reading before the barrier above.
        if constexpr (FB == 1) SC_WAIT_LGKM0();
        // the next tap's row numbers are spread and tap k+2 looked up after the first
        // group's MFMAs: ahead of them, their LDS round trips held the start of every tap
        int32_t jnext[NGP];
        // the copies go out in the first half of the groups, so they have half a tap to
        // land before the wait at its end
        constexpr int P = PF ? NWP + NGP : 0, GP = G >= 2 ? G / 2 : 1;
        // A fragments of group g are read during group g - 1 (the groups are kept
        // apart, so nothing else would hide the LDS latency in front of the MFMAs)
        auto read_a = [&](int g, uint4 (&a)[RT]) {
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const int o = 32 * (og * RT + r) + l32;
                a[r] = *(const uint4 *)(wb + o * RB + (((2 * g + half) ^ swz<RB>(o)) << 4));
            }
        };
        uint4 A[2][RT];
        read_a(0, A[0]);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            __builtin_amdgcn_sched_barrier(0);  // keep each group's copies in place
            if (g + 1 < G) read_a(g + 1, A[(g + 1) & 1]);
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
                for (int t = 0; t < VT; ++t) Mma<T>::step(acc[r][t], A[g & 1][r], F[t][g]);
            if constexpr (PF) {
                if (g == 0) {
                    spread_rows(row_of(jn), jnext);
                    jn = lookup(k + 2 < 27 ? k + 2 : 26);
                }
            }
#pragma unroll
            for (int p = g * P / GP; p < (g < GP ? (g + 1) * P / GP : 0); ++p) {
                if (p < NWP) copy_w_piece(k + 1, wnxt, p);
                else gather_piece(jnext, fnxt, p - NWP);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int k = 0; k < 26; k += 2) {
        step(std::false_type{}, std::true_type{}, k);
        step(std::true_type{}, std::true_type{}, k + 1);
    }
    step(std::false_type{}, std::false_type{}, 26);

#pragma unroll
    for (int t = 0; t < VT; ++t) {
        const int64_t v = vbase + 32 * t + l32;
        if (v >= n) continue;
        const int64_t orow = perm[v];
        if ((uint64_t)orow >= (uint64_t)n) continue;
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int o = 32 * (og * RT + r) + 8 * q + 4 * half;
                float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
                if (bias) b = *(const float4 *)(bias + o);
                Store4<T>::put(out + orow * COUT + o, acc[r][t][4 * q] + b.x, acc[r][t][4 * q + 1] + b.y,
                               acc[r][t][4 * q + 2] + b.z, acc[r][t][4 * q + 3] + b.w);
            }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static bool pow2_le32(int c) { return c == 1 || c == 2 || c == 4 || c == 8 || c == 16 || c == 32; }
static bool mfma_size(int c) { return c == 32 || c == 64 || c == 128; }

template <typename T>
static int launch_generic(const void *feats, const void *w, const float *bias, const int32_t *nbr,
                          const int32_t *perm, void *out, int64_t n, int cin, int cout, int flip,
                          hipStream_t s)
{
    const int64_t total = n * cout;
    const unsigned grid = (unsigned)((total + 255) / 256);
    hipLaunchKernelGGL(k_conv_generic<T>, dim3(grid), dim3(256), 0, s, (const T *)feats,
                       (const T *)w, bias, nbr, perm, (T *)out, n, cin, cout, flip);
    SC_LAUNCHED("conv_generic");
    return SUBMCONV_OK;
}

template <typename T, int CIN, int COUT>
static int launch_lowc_t(const void *feats, const void *w, const float *bias, const int32_t *nbr,
                         const int32_t *perm, void *out, int64_t n, int flip, hipStream_t s)
{
    constexpr int VPB = 256 / COUT;
    int64_t blocks = (n + VPB - 1) / VPB;
    if (blocks > 2048) blocks = 2048;  // grid-stride beyond: amortises the weight staging
    hipLaunchKernelGGL((k_conv_lowc<T, CIN, COUT>), dim3((unsigned)blocks), dim3(256), 0, s,
                       (const T *)feats, (const T *)w, bias, nbr, perm, (T *)out, n, flip);
    SC_LAUNCHED("conv_lowc");
    return SUBMCONV_OK;
}

template <typename T, int CIN>
static int launch_lowc_cout(const void *f, const void *w, const float *b, const int32_t *nbr, const int32_t *perm,
                            void *o, int64_t n, int cout, int flip, hipStream_t s)
{
    switch (cout) {
    case 1: return launch_lowc_t<T, CIN, 1>(f, w, b, nbr, perm, o, n, flip, s);
    case 2: return launch_lowc_t<T, CIN, 2>(f, w, b, nbr, perm, o, n, flip, s);
    case 4: return launch_lowc_t<T, CIN, 4>(f, w, b, nbr, perm, o, n, flip, s);
    case 8: return launch_lowc_t<T, CIN, 8>(f, w, b, nbr, perm, o, n, flip, s);
    case 16: return launch_lowc_t<T, CIN, 16>(f, w, b, nbr, perm, o, n, flip, s);
    case 32: return launch_lowc_t<T, CIN, 32>(f, w, b, nbr, perm, o, n, flip, s);
    }
    return fail(SUBMCONV_E_UNSUPPORTED, "lowc kernel: Cout must be a power of two <= 32");
}

template <typename T>
static int launch_lowc(const void *f, const void *w, const float *b, const int32_t *nbr, const int32_t *perm, void *o,
                       int64_t n, int cin, int cout, int flip, hipStream_t s)
{
    switch (cin) {
    case 1: return launch_lowc_cout<T, 1>(f, w, b, nbr, perm, o, n, cout, flip, s);
    case 2: return launch_lowc_cout<T, 2>(f, w, b, nbr, perm, o, n, cout, flip, s);
    case 4: return launch_lowc_cout<T, 4>(f, w, b, nbr, perm, o, n, cout, flip, s);
    case 8: return launch_lowc_cout<T, 8>(f, w, b, nbr, perm, o, n, cout, flip, s);
    case 16: return launch_lowc_cout<T, 16>(f, w, b, nbr, perm, o, n, cout, flip, s);
    case 32: return launch_lowc_cout<T, 32>(f, w, b, nbr, perm, o, n, cout, flip, s);
    }
    return fail(SUBMCONV_E_UNSUPPORTED, "lowc kernel: Cin must be a power of two <= 32");
}

// compute units of the current device (cached per device)
static int current_device_cus()
{
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (dev >= 0 && dev < 64 && cached[dev]) return cached[dev];
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (dev >= 0 && dev < 64) cached[dev] = cus;
    return cus;
}

template <typename T, int CIN, int COUT, int VT>
static void launch_mfma_vt(const void *f, const void *w, const float *b, const int32_t *nbr, const int32_t *perm,
                           void *o, int64_t n, int flip, hipStream_t s)
{
    if constexpr (RowShape<T, CIN, COUT, VT>::LDS <= 160 * 1024) {
        // Split Cout over two waves per column when one-wave columns would leave
        // fewer than two blocks per CU (256 CUs).
        constexpr int per_block = RowShape<T, CIN, COUT, VT>::VOX_PER_BLOCK;
        if constexpr (VT == 1 && COUT >= 64) {
            if constexpr (RowShape<T, CIN, COUT, 1, 2>::LDS <= 160 * 1024) {
                if ((n + per_block - 1) / per_block < 2 * 256) {
                    constexpr int pb2 = RowShape<T, CIN, COUT, 1, 2>::VOX_PER_BLOCK;
                    const unsigned grid = (unsigned)((n + pb2 - 1) / pb2);
                    hipLaunchKernelGGL((k_conv_mfma_rows<T, CIN, COUT, 1, 2>), dim3(grid), dim3(256), 0, s,
                                       (const T *)f, (const T *)w, b, nbr, perm, (T *)o, n, flip);
                    return;
                }
            }
        }
        const unsigned grid = (unsigned)((n + per_block - 1) / per_block);
        hipLaunchKernelGGL((k_conv_mfma_rows<T, CIN, COUT, VT, 1>), dim3(grid), dim3(256), 0, s,
                           (const T *)f, (const T *)w, b, nbr, perm, (T *)o, n, flip);
    } else {
        // persistent: one block per CU (fewer when there are fewer 32-voxel columns)
        const int64_t ncols = (n + 31) / 32;
        const int64_t cus = current_device_cus();
        const unsigned grid = (unsigned)(ncols < cus ? ncols : cus);
        hipLaunchKernelGGL((k_conv_mfma<T, CIN, COUT, VT>), dim3(grid), dim3(64 * MFMA_P_WAVES), 0, s,
                           (const T *)f, (const T *)w, b, nbr, perm, (T *)o, n, flip);
    }
}

template <typename T, int CIN, int COUT>
static int launch_mfma_tt(const void *f, const void *w, const float *b, const int32_t *nbr, const int32_t *perm, void *o,
                          int64_t n, int flip, hipStream_t s)
{
    // Two 32-voxel columns per wave share each weight fragment, except at fp32 with
    // 128 channels (registers) and on small sets, where 64 voxels per wave would
    // leave most CUs without a block (256 voxels per block; 2 blocks per CU wanted).
    constexpr bool one = sizeof(T) == 4 && (CIN >= 128 || COUT >= 128);
    if (one || n < (int64_t)256 * 2 * 256)
        launch_mfma_vt<T, CIN, COUT, 1>(f, w, b, nbr, perm, o, n, flip, s);
    else
        launch_mfma_vt<T, CIN, COUT, (one ? 1 : 2)>(f, w, b, nbr, perm, o, n, flip, s);
    SC_LAUNCHED("conv_mfma");
    return SUBMCONV_OK;
}

template <int CIN, int COUT>
static int launch_mfma_t(const void *f, const void *w, const float *b, const int32_t *nbr, const int32_t *perm, void *o,
                         int64_t n, int dtype, int flip, hipStream_t s)
{
    if (dtype == SUBMCONV_BF16) return launch_mfma_tt<uint16_t, CIN, COUT>(f, w, b, nbr, perm, o, n, flip, s);
    return launch_mfma_tt<float, CIN, COUT>(f, w, b, nbr, perm, o, n, flip, s);
}

template <int CIN>
static int launch_mfma_cout(const void *f, const void *w, const float *b, const int32_t *nbr, const int32_t *perm,
                            void *o, int64_t n, int cout, int dtype, int flip, hipStream_t s)
{
    switch (cout) {
    case 32: return launch_mfma_t<CIN, 32>(f, w, b, nbr, perm, o, n, dtype, flip, s);
    case 64: return launch_mfma_t<CIN, 64>(f, w, b, nbr, perm, o, n, dtype, flip, s);
    case 128: return launch_mfma_t<CIN, 128>(f, w, b, nbr, perm, o, n, dtype, flip, s);
    }
    return fail(SUBMCONV_E_UNSUPPORTED, "mfma kernel: Cout must be 32, 64 or 128");
}

static int launch_mfma(const void *f, const void *w, const float *b, const int32_t *nbr, const int32_t *perm, void *o,
                       int64_t n, int cin, int cout, int dtype, int flip, hipStream_t s)
{
    if (cin == 16 || cout == 16) {
        if (!mfma16_supported(cin, cout, dtype, n))
            return fail(SUBMCONV_E_UNSUPPORTED, "mfma kernel: 16 channels need Cin = Cout = 16 and N * 16 * %d <= 2^31 - 1",
                        dtype == SUBMCONV_F32 ? 4 : 2);
        if (dtype == SUBMCONV_BF16) launch_mfma16_t<uint16_t>(f, w, b, nbr, perm, o, n, flip, s);
        else launch_mfma16_t<float>(f, w, b, nbr, perm, o, n, flip, s);
        SC_LAUNCHED("conv_mfma16");
        return SUBMCONV_OK;
    }
    switch (cin) {
    case 32: return launch_mfma_cout<32>(f, w, b, nbr, perm, o, n, cout, dtype, flip, s);
    case 64: return launch_mfma_cout<64>(f, w, b, nbr, perm, o, n, cout, dtype, flip, s);
    case 128: return launch_mfma_cout<128>(f, w, b, nbr, perm, o, n, cout, dtype, flip, s);
    }
    return fail(SUBMCONV_E_UNSUPPORTED, "mfma kernel: Cin must be 16, 32, 64 or 128");
}

bool window_supported(int cin, int cout, int dtype, int64_t n);
bool big_supported(int cin, int cout, int dtype, int64_t n);
int launch_big(const void *feats, const void *w, const float *bias, const submconv_rulebook *rb, void *out,
               int cin, int cout, int dtype, int flip, hipStream_t s);
int launch_window(const void *feats, const void *w, const float *bias, const submconv_rulebook *rb,
                  void *out, int cin, int cout, int dtype, int flip, hipStream_t s);

int choose_forward_kernel(int cin, int cout, int dtype, int64_t n)
{
    if (window_supported(cin, cout, dtype, n)) return SUBMCONV_KERNEL_WINDOW;
    // bf16 64 -> 64 on large sets: the row-gathered kernel (64 voxels per column, whole
    // rows through LDS) measured 5-6% faster than the persistent one at 1.19M voxels, and
    // 8% slower at 49k (32-voxel columns split in Cout there)
    if (dtype == SUBMCONV_BF16 && cin == 64 && cout == 64 && n >= (int64_t(1) << 19)) return SUBMCONV_KERNEL_MFMA;
    if (big_supported(cin, cout, dtype, n)) return SUBMCONV_KERNEL_PERSISTENT;
    if (mfma_size(cin) && mfma_size(cout)) return SUBMCONV_KERNEL_MFMA;
    // 16 -> 16 on the matrix cores: 8.0 us against 27.3 us for the shuffle kernel on the
    // 450-voxel 16^3 sphere (whose 27 x 16 unrolled shuffles the compiler serialises)
    if (mfma16_supported(cin, cout, dtype, n)) return SUBMCONV_KERNEL_MFMA;
    if (pow2_le32(cin) && pow2_le32(cout)) return SUBMCONV_KERNEL_LOWC;
    (void)dtype;
    return SUBMCONV_KERNEL_GENERIC;
}

int launch_forward(const void *feats, const void *w, const float *bias, const submconv_rulebook *rb,
                   void *out, int cin, int cout, int dtype, int flip, int variant, hipStream_t s)
{
    const int64_t n = rb->n;
    const int32_t *nbr = rb->nbr_sp, *perm = rb->perm;
    if (n == 0) return SUBMCONV_OK;
    if (variant == SUBMCONV_KERNEL_AUTO) variant = choose_forward_kernel(cin, cout, dtype, n);
    switch (variant) {
    case SUBMCONV_KERNEL_GENERIC:
        return dtype == SUBMCONV_F32
                   ? launch_generic<float>(feats, w, bias, nbr, perm, out, n, cin, cout, flip, s)
                   : launch_generic<uint16_t>(feats, w, bias, nbr, perm, out, n, cin, cout, flip, s);
    case SUBMCONV_KERNEL_LOWC:
        return dtype == SUBMCONV_F32
                   ? launch_lowc<float>(feats, w, bias, nbr, perm, out, n, cin, cout, flip, s)
                   : launch_lowc<uint16_t>(feats, w, bias, nbr, perm, out, n, cin, cout, flip, s);
    case SUBMCONV_KERNEL_MFMA:
        return launch_mfma(feats, w, bias, nbr, perm, out, n, cin, cout, dtype, flip, s);
    case SUBMCONV_KERNEL_WINDOW:
        return launch_window(feats, w, bias, rb, out, cin, cout, dtype, flip, s);
    case SUBMCONV_KERNEL_PERSISTENT:
        return launch_big(feats, w, bias, rb, out, cin, cout, dtype, flip, s);
    }
    return fail(SUBMCONV_E_INVALID_ARG, "unknown forward kernel variant %d", variant);
}

}  // namespace sc
