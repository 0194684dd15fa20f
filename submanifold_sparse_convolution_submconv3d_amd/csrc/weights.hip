// Weight layouts of a 3x3x3 kernel (lato.2_mrp_mlx working notes, "Key facts":
// spconv stores KRSC [out, kz, ky, kx, in], torch Conv3d [out, in, kz, ky, kx]; both
// are 5-D, so the rank does not tell them apart and misreading one for the other
// keeps every shape valid).  The forward kernels take KRSC; this file classifies a
// 5-D shape and converts either layout to KRSC, optionally mirrored (tap k -> 26 - k,
// the kernel the flip option stands for: same page, "Unresolved").
#include "common.h"

namespace sc {

// dst[o, k, c] = src[o, k', c] (KRSC) or src[o, c, k'] (Conv3d), k' = flip ? 26 - k : k;
// one thread per destination element.
template <typename T>
__global__ __launch_bounds__(256) void k_weight_convert(const T *__restrict__ src, int layout, int cout, int cin,
                                                        int flip, T *__restrict__ dst)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)cout * 27 * cin;
    if (e >= total) return;
    const int c = (int)(e % cin);
    const int64_t ok = e / cin;
    const int k = (int)(ok % 27), o = (int)(ok / 27);
    const int ks = flip ? 26 - k : k;
    const int64_t si = layout == SUBMCONV_LAYOUT_KRSC ? ((int64_t)o * 27 + ks) * cin + c
                                                      : ((int64_t)o * cin + c) * 27 + ks;
    dst[e] = src[si];
}

int classify_5d(const int64_t *shape, int hint, int *layout)
{
    for (int i = 0; i < 5; ++i)
        if (shape[i] < 1) return fail(SUBMCONV_E_INVALID_ARG, "shape[%d] = %lld", i, (long long)shape[i]);
    const bool krsc = shape[1] == 3 && shape[2] == 3 && shape[3] == 3;
    const bool oidhw = shape[2] == 3 && shape[3] == 3 && shape[4] == 3;
    if (hint != SUBMCONV_LAYOUT_UNKNOWN && hint != SUBMCONV_LAYOUT_KRSC && hint != SUBMCONV_LAYOUT_OIDHW)
        return fail(SUBMCONV_E_INVALID_ARG, "hint %d", hint);
    if (!krsc && !oidhw)
        return fail(SUBMCONV_E_UNSUPPORTED, "shape [%lld,%lld,%lld,%lld,%lld] is not a 3x3x3 kernel in either layout",
                    (long long)shape[0], (long long)shape[1], (long long)shape[2], (long long)shape[3],
                    (long long)shape[4]);
    if (krsc && oidhw) {  // [O,3,3,3,3]: both readings fit; only the caller's module knows
        if (hint == SUBMCONV_LAYOUT_UNKNOWN)
            return fail(SUBMCONV_E_INVALID_ARG, "shape [%lld,3,3,3,3] fits both layouts: pass the layout the module implies",
                        (long long)shape[0]);
        *layout = hint;
        return SUBMCONV_OK;
    }
    const int found = krsc ? SUBMCONV_LAYOUT_KRSC : SUBMCONV_LAYOUT_OIDHW;
    if (hint != SUBMCONV_LAYOUT_UNKNOWN && hint != found)
        return fail(SUBMCONV_E_INVALID_ARG, "the shape is %s but the hint says otherwise",
                    found == SUBMCONV_LAYOUT_KRSC ? "KRSC" : "Conv3d [O,I,kz,ky,kx]");
    *layout = found;
    return SUBMCONV_OK;
}

int weight_convert(const void *src, int layout, int cout, int cin, int dtype, int flip, void *dst, hipStream_t s)
{
    const int64_t total = (int64_t)cout * 27 * cin;
    const unsigned grid = (unsigned)((total + 255) / 256);
    if (dtype == SUBMCONV_F32)
        hipLaunchKernelGGL(k_weight_convert<float>, dim3(grid), dim3(256), 0, s, (const float *)src, layout, cout,
                           cin, flip, (float *)dst);
    else
        hipLaunchKernelGGL(k_weight_convert<uint16_t>, dim3(grid), dim3(256), 0, s, (const uint16_t *)src, layout,
                           cout, cin, flip, (uint16_t *)dst);
    SC_LAUNCHED("weight_convert");
    return SUBMCONV_OK;
}

}  // namespace sc
