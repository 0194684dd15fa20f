// Forward kernels of the submanifold 3x3x3 convolution.
//
//   out[i, o] = bias[o] + sum_k sum_c W[o, k', c] * feats[nbr[i, k], c]
//
// over the taps k with nbr[i, k] >= 0, k' = k (correlation) or 26 - k (the
// mirrored kernel), W in KRSC layout [Cout, 27, Cin] (lato.2_mrp_mlx working
// notes, "Key facts" for the layout, commit summary for the mirror flag).
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
                                                      T *__restrict__ out, int64_t n, int cin,
                                                      int cout, int flip)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t i = idx / cout;
    const int o = (int)(idx - i * cout);
    if (i >= n) return;
    float acc = 0.f;
    for (int k = 0; k < 27; ++k) {
        const int32_t j = nbr[i * 27 + k];
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
                                                   T *__restrict__ out, int64_t n, int flip)
{
    static_assert(COUT <= 64 && (64 % COUT) == 0, "group must divide the wave");
    constexpr int VPB = 256 / COUT;                         // voxels per block pass
    constexpr int PER = (CIN + COUT - 1) / COUT;            // feature elements per lane
    __shared__ float s_w[27 * CIN * COUT];                  // [27][CIN][COUT]
    for (int e = threadIdx.x; e < 27 * CIN * COUT; e += 256) {
        const int o = e % COUT, c = (e / COUT) % CIN, k = e / (COUT * CIN);
        s_w[e] = Elem<T>::to_f32(w[((int64_t)o * 27 + k) * CIN + c]);
    }
    __syncthreads();
    const int o = threadIdx.x % COUT;
    const int lane = threadIdx.x & 63;
    const int gbase = lane - (lane % COUT);                 // first lane of this voxel's group
    const float b = bias ? bias[o] : 0.f;
    const int64_t stride = (int64_t)gridDim.x * VPB;
    // every lane of a wave runs the same number of iterations (shuffles need all lanes)
    for (int64_t i0 = (int64_t)blockIdx.x * VPB; i0 < n; i0 += stride) {
        const int64_t i = i0 + threadIdx.x / COUT;
        const bool live = i < n;
        float acc = 0.f;
        for (int k = 0; k < 27; ++k) {
            int32_t j = live ? nbr[i * 27 + k] : -1;
            if ((uint32_t)j >= (uint64_t)n) j = -1;
            float f[PER];
#pragma unroll
            for (int m = 0; m < PER; ++m) {
                const int c = o + m * COUT;
                f[m] = (j >= 0 && c < CIN) ? Elem<T>::to_f32(feats[(int64_t)j * CIN + c]) : 0.f;
            }
            const float *wk = s_w + (flip ? 26 - k : k) * CIN * COUT + o;
#pragma unroll
            for (int c = 0; c < CIN; ++c) {
                const float fc = __shfl(f[c / COUT], gbase + (c % COUT), 64);
                acc = fmaf(wk[c * COUT], fc, acc);
            }
        }
        if (live) out[i * COUT + o] = Elem<T>::from_f32(acc + b);
    }
}

// ---------------------------------------------------------------------------
// mfma, bf16: v_mfma_f32_32x32x16_bf16
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) .. +7
//   B (16 x 32): lane l holds column l%32, k = 8*(l/32) .. +7
//   D (32 x 32): lane l holds column l%32, rows 8*(r/4) + 4*(l/32) + r%4, r = 0..15
// ---------------------------------------------------------------------------

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t *p)
{
    const uint4 v = *(const uint4 *)p;
    return __builtin_bit_cast(bf16x8_t, v);
}

template <int CIN, int COUT, int VT>
__global__ __launch_bounds__(256) void k_conv_mfma_bf16(const uint16_t *__restrict__ feats,
                                                        const uint16_t *__restrict__ w,
                                                        const float *__restrict__ bias,
                                                        const int32_t *__restrict__ nbr,
                                                        uint16_t *__restrict__ out, int64_t n,
                                                        int flip)
{
    constexpr int RT = COUT / 32;  // row tiles (output channels)
    constexpr int KS = CIN / 16;   // k steps per tap
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t vbase = ((int64_t)blockIdx.x * 4 + wave) * (VT * 32);

    floatx16 acc[RT][VT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int t = 0; t < VT; ++t)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[r][t][q] = 0.f;

    for (int k = 0; k < 27; ++k) {
        int32_t j[VT];
        bool any = false;
#pragma unroll
        for (int t = 0; t < VT; ++t) {
            const int64_t v = vbase + 32 * t + l32;
            j[t] = v < n ? nbr[v * 27 + k] : -1;
            if ((uint32_t)j[t] >= (uint64_t)n) j[t] = -1;
            any |= j[t] >= 0;
        }
        if (!__any(any)) continue;  // wave-uniform
        const int kw = flip ? 26 - k : k;
        bf16x8_t bf[VT][KS];
#pragma unroll
        for (int t = 0; t < VT; ++t)
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                if (j[t] >= 0) bf[t][s] = load_bf16x8(feats + (int64_t)j[t] * CIN + 16 * s + 8 * half);
                else bf[t][s] = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
            }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const uint16_t *wr = w + ((int64_t)(32 * r + l32) * 27 + kw) * CIN + 8 * half;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const bf16x8_t a = load_bf16x8(wr + 16 * s);
#pragma unroll
                for (int t = 0; t < VT; ++t)
                    acc[r][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bf[t][s], acc[r][t], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < VT; ++t) {
        const int64_t v = vbase + 32 * t + l32;
        if (v >= n) continue;
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int o = 32 * r + 8 * g + 4 * half;
                float b0 = 0.f, b1 = 0.f, b2 = 0.f, b3 = 0.f;
                if (bias) { b0 = bias[o]; b1 = bias[o + 1]; b2 = bias[o + 2]; b3 = bias[o + 3]; }
                const uint32_t lo = (uint32_t)f32_to_bf16(acc[r][t][4 * g] + b0) |
                                    ((uint32_t)f32_to_bf16(acc[r][t][4 * g + 1] + b1) << 16);
                const uint32_t hi = (uint32_t)f32_to_bf16(acc[r][t][4 * g + 2] + b2) |
                                    ((uint32_t)f32_to_bf16(acc[r][t][4 * g + 3] + b3) << 16);
                *(uint2 *)(out + v * COUT + o) = make_uint2(lo, hi);
            }
    }
}

// ---------------------------------------------------------------------------
// mfma, fp32: v_mfma_f32_32x32x2_f32
//   A (32 x 2): lane l holds row l%32, k = l/32; B likewise with column l%32.
//   The contraction index may be permuted as long as A and B agree: lane half h
//   loads channels [8g + 4h, 8g + 4h + 4) and feeds element e in step e, so the
//   four steps of group g cover channels 8g .. 8g+7 once each.
// ---------------------------------------------------------------------------

template <int CIN, int COUT, int VT>
__global__ __launch_bounds__(256) void k_conv_mfma_f32(const float *__restrict__ feats,
                                                       const float *__restrict__ w,
                                                       const float *__restrict__ bias,
                                                       const int32_t *__restrict__ nbr,
                                                       float *__restrict__ out, int64_t n, int flip)
{
    constexpr int RT = COUT / 32;
    constexpr int KG = CIN / 8;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t vbase = ((int64_t)blockIdx.x * 4 + wave) * (VT * 32);

    floatx16 acc[RT][VT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int t = 0; t < VT; ++t)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[r][t][q] = 0.f;

    for (int k = 0; k < 27; ++k) {
        int32_t j[VT];
        bool any = false;
#pragma unroll
        for (int t = 0; t < VT; ++t) {
            const int64_t v = vbase + 32 * t + l32;
            j[t] = v < n ? nbr[v * 27 + k] : -1;
            if ((uint32_t)j[t] >= (uint64_t)n) j[t] = -1;
            any |= j[t] >= 0;
        }
        if (!__any(any)) continue;
        const int kw = flip ? 26 - k : k;
#pragma unroll
        for (int g = 0; g < KG; ++g) {
            float4 bf[VT];
#pragma unroll
            for (int t = 0; t < VT; ++t)
                bf[t] = j[t] >= 0 ? *(const float4 *)(feats + (int64_t)j[t] * CIN + 8 * g + 4 * half)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const float4 a = *(const float4 *)(w + ((int64_t)(32 * r + l32) * 27 + kw) * CIN + 8 * g + 4 * half);
#pragma unroll
                for (int t = 0; t < VT; ++t) {
                    acc[r][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, bf[t].x, acc[r][t], 0, 0, 0);
                    acc[r][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, bf[t].y, acc[r][t], 0, 0, 0);
                    acc[r][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, bf[t].z, acc[r][t], 0, 0, 0);
                    acc[r][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, bf[t].w, acc[r][t], 0, 0, 0);
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < VT; ++t) {
        const int64_t v = vbase + 32 * t + l32;
        if (v >= n) continue;
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int o = 32 * r + 8 * g + 4 * half;
                float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
                if (bias) b = *(const float4 *)(bias + o);
                *(float4 *)(out + v * COUT + o) =
                    make_float4(acc[r][t][4 * g] + b.x, acc[r][t][4 * g + 1] + b.y,
                                acc[r][t][4 * g + 2] + b.z, acc[r][t][4 * g + 3] + b.w);
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
                          void *out, int64_t n, int cin, int cout, int flip, hipStream_t s)
{
    const int64_t total = n * cout;
    const unsigned grid = (unsigned)((total + 255) / 256);
    hipLaunchKernelGGL(k_conv_generic<T>, dim3(grid), dim3(256), 0, s, (const T *)feats,
                       (const T *)w, bias, nbr, (T *)out, n, cin, cout, flip);
    SC_LAUNCHED("conv_generic");
    return SUBMCONV_OK;
}

template <typename T, int CIN, int COUT>
static int launch_lowc_t(const void *feats, const void *w, const float *bias, const int32_t *nbr,
                         void *out, int64_t n, int flip, hipStream_t s)
{
    constexpr int VPB = 256 / COUT;
    int64_t blocks = (n + VPB - 1) / VPB;
    if (blocks > 2048) blocks = 2048;  // grid-stride beyond: amortises the weight staging
    hipLaunchKernelGGL((k_conv_lowc<T, CIN, COUT>), dim3((unsigned)blocks), dim3(256), 0, s,
                       (const T *)feats, (const T *)w, bias, nbr, (T *)out, n, flip);
    SC_LAUNCHED("conv_lowc");
    return SUBMCONV_OK;
}

template <typename T, int CIN>
static int launch_lowc_cout(const void *f, const void *w, const float *b, const int32_t *nbr,
                            void *o, int64_t n, int cout, int flip, hipStream_t s)
{
    switch (cout) {
    case 1: return launch_lowc_t<T, CIN, 1>(f, w, b, nbr, o, n, flip, s);
    case 2: return launch_lowc_t<T, CIN, 2>(f, w, b, nbr, o, n, flip, s);
    case 4: return launch_lowc_t<T, CIN, 4>(f, w, b, nbr, o, n, flip, s);
    case 8: return launch_lowc_t<T, CIN, 8>(f, w, b, nbr, o, n, flip, s);
    case 16: return launch_lowc_t<T, CIN, 16>(f, w, b, nbr, o, n, flip, s);
    case 32: return launch_lowc_t<T, CIN, 32>(f, w, b, nbr, o, n, flip, s);
    }
    return fail(SUBMCONV_E_UNSUPPORTED, "lowc kernel: Cout must be a power of two <= 32");
}

template <typename T>
static int launch_lowc(const void *f, const void *w, const float *b, const int32_t *nbr, void *o,
                       int64_t n, int cin, int cout, int flip, hipStream_t s)
{
    switch (cin) {
    case 1: return launch_lowc_cout<T, 1>(f, w, b, nbr, o, n, cout, flip, s);
    case 2: return launch_lowc_cout<T, 2>(f, w, b, nbr, o, n, cout, flip, s);
    case 4: return launch_lowc_cout<T, 4>(f, w, b, nbr, o, n, cout, flip, s);
    case 8: return launch_lowc_cout<T, 8>(f, w, b, nbr, o, n, cout, flip, s);
    case 16: return launch_lowc_cout<T, 16>(f, w, b, nbr, o, n, cout, flip, s);
    case 32: return launch_lowc_cout<T, 32>(f, w, b, nbr, o, n, cout, flip, s);
    }
    return fail(SUBMCONV_E_UNSUPPORTED, "lowc kernel: Cin must be a power of two <= 32");
}

template <int CIN, int COUT>
static int launch_mfma_t(const void *f, const void *w, const float *b, const int32_t *nbr, void *o,
                         int64_t n, int dtype, int flip, hipStream_t s)
{
    if (dtype == SUBMCONV_BF16) {
        constexpr int VT = (COUT >= 128) ? 2 : 2;
        const int64_t per_block = 4 * 32 * VT;
        const unsigned grid = (unsigned)((n + per_block - 1) / per_block);
        hipLaunchKernelGGL((k_conv_mfma_bf16<CIN, COUT, VT>), dim3(grid), dim3(256), 0, s,
                           (const uint16_t *)f, (const uint16_t *)w, b, nbr, (uint16_t *)o, n, flip);
    } else {
        constexpr int VT = 1;
        const int64_t per_block = 4 * 32 * VT;
        const unsigned grid = (unsigned)((n + per_block - 1) / per_block);
        hipLaunchKernelGGL((k_conv_mfma_f32<CIN, COUT, VT>), dim3(grid), dim3(256), 0, s,
                           (const float *)f, (const float *)w, b, nbr, (float *)o, n, flip);
    }
    SC_LAUNCHED("conv_mfma");
    return SUBMCONV_OK;
}

template <int CIN>
static int launch_mfma_cout(const void *f, const void *w, const float *b, const int32_t *nbr,
                            void *o, int64_t n, int cout, int dtype, int flip, hipStream_t s)
{
    switch (cout) {
    case 32: return launch_mfma_t<CIN, 32>(f, w, b, nbr, o, n, dtype, flip, s);
    case 64: return launch_mfma_t<CIN, 64>(f, w, b, nbr, o, n, dtype, flip, s);
    case 128: return launch_mfma_t<CIN, 128>(f, w, b, nbr, o, n, dtype, flip, s);
    }
    return fail(SUBMCONV_E_UNSUPPORTED, "mfma kernel: Cout must be 32, 64 or 128");
}

static int launch_mfma(const void *f, const void *w, const float *b, const int32_t *nbr, void *o,
                       int64_t n, int cin, int cout, int dtype, int flip, hipStream_t s)
{
    switch (cin) {
    case 32: return launch_mfma_cout<32>(f, w, b, nbr, o, n, cout, dtype, flip, s);
    case 64: return launch_mfma_cout<64>(f, w, b, nbr, o, n, cout, dtype, flip, s);
    case 128: return launch_mfma_cout<128>(f, w, b, nbr, o, n, cout, dtype, flip, s);
    }
    return fail(SUBMCONV_E_UNSUPPORTED, "mfma kernel: Cin must be 32, 64 or 128");
}

int choose_forward_kernel(int cin, int cout, int dtype)
{
    if (mfma_size(cin) && mfma_size(cout)) return SUBMCONV_KERNEL_MFMA;
    if (pow2_le32(cin) && pow2_le32(cout)) return SUBMCONV_KERNEL_LOWC;
    (void)dtype;
    return SUBMCONV_KERNEL_GENERIC;
}

int launch_forward(const void *feats, const void *w, const float *bias, const int32_t *nbr,
                   void *out, int64_t n, int cin, int cout, int dtype, int flip, int variant,
                   hipStream_t s)
{
    if (n == 0) return SUBMCONV_OK;
    if (variant == SUBMCONV_KERNEL_AUTO) variant = choose_forward_kernel(cin, cout, dtype);
    switch (variant) {
    case SUBMCONV_KERNEL_GENERIC:
        return dtype == SUBMCONV_F32
                   ? launch_generic<float>(feats, w, bias, nbr, out, n, cin, cout, flip, s)
                   : launch_generic<uint16_t>(feats, w, bias, nbr, out, n, cin, cout, flip, s);
    case SUBMCONV_KERNEL_LOWC:
        return dtype == SUBMCONV_F32
                   ? launch_lowc<float>(feats, w, bias, nbr, out, n, cin, cout, flip, s)
                   : launch_lowc<uint16_t>(feats, w, bias, nbr, out, n, cin, cout, flip, s);
    case SUBMCONV_KERNEL_MFMA:
        return launch_mfma(feats, w, bias, nbr, out, n, cin, cout, dtype, flip, s);
    }
    return fail(SUBMCONV_E_INVALID_ARG, "unknown forward kernel variant %d", variant);
}

}  // namespace sc
