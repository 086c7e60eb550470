// attend_inst.hip -- instances of the split kernel for one (K type, V type)
// pair.  Built once per pair with -DRKV_KT=<t> -DRKV_VT=<t> (0 f32, 1 f16,
// 2 q8_0, 3 q4_0, 4 TBQ3) so that the instances compile in parallel.
#include "attend_kernel.h"
#include "attend_shd.h"

#if !defined(RKV_KT) || !defined(RKV_VT)
#error "RKV_KT and RKV_VT must be defined"
#endif
#if RKV_KT == 1 && RKV_VT == 1
#include "attend_rgs.h"  // (its kernel is not a template: one unit defines it)
#endif

#define RKV_CAT4(a, b, c, d) a##b##c##d
#define RKV_NAME(kt, vt) RKV_CAT4(launch_split_k, kt, _v, vt)

namespace rkv {

// Block-type K and V at head_dim 256 / 512 run as 2 / 4 dim slices of 128
// (see rkv_split_kernel): the instance used for a requested head_dim.
constexpr bool kBlockKV = (RKV_KT == kQ8 || RKV_KT == kQ4) && (RKV_VT == kQ8 || RKV_VT == kQ4 || RKV_VT == kT3);
template <int D>
constexpr int slices_of() { return kBlockKV && D > 128 ? D / 128 : 1; }
// An instance exists for the head_dim (TBQ3 values come in blocks of 128;
// an f32 row of 512 values does not fit the LDS tile).
template <int D>
constexpr bool has_instance() { return !(RKV_VT == kT3 && D % 128) && !(D == 512 && (RKV_KT == kF32 || RKV_VT == kF32)); }

template <int D, int RT>
static hipError_t go(dim3 grid, const float *q, float *pa, float2 *pm, float *o, float *lse, const SplitParams &p,
                     hipStream_t stream)
{
    if constexpr (!has_instance<D>()) {
        return hipErrorInvalidValue;
    } else if constexpr (slices_of<D>() > 1) {
        constexpr int DS = slices_of<D>();
        hipLaunchKernelGGL((rkv_split_kernel<RKV_KT, RKV_VT, 128, RT, DS>), grid,
                           dim3(64 * Shape<RKV_KT, RKV_VT, 128>::waves(sp_rows(RT, DS))), 0, stream, q, pa, pm, o, lse, p);
        return hipGetLastError();
    } else {
        hipLaunchKernelGGL((rkv_split_kernel<RKV_KT, RKV_VT, D, RT>), grid, dim3(64 * Shape<RKV_KT, RKV_VT, D>::waves(RT)), 0,
                           stream, q, pa, pm, o, lse, p);
        return hipGetLastError();
    }
}

template <int D>
static hipError_t by_rt(int rt, dim3 grid, const float *q, float *pa, float2 *pm, float *o, float *lse,
                        const SplitParams &p, hipStream_t s)
{
    switch (rt) {
    case 1: return go<D, 1>(grid, q, pa, pm, o, lse, p, s);
    case 2: return go<D, 2>(grid, q, pa, pm, o, lse, p, s);
    case 4: return go<D, 4>(grid, q, pa, pm, o, lse, p, s);
    case 5: return go<D, 5>(grid, q, pa, pm, o, lse, p, s);
    case 8: return go<D, 8>(grid, q, pa, pm, o, lse, p, s);
    case 16: return go<D, 16>(grid, q, pa, pm, o, lse, p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t RKV_NAME(RKV_KT, RKV_VT)(int d, int rt, dim3 grid, const float *q, float *pa, float2 *pm, float *o,
                                    float *lse, const SplitParams &p, hipStream_t s)
{
    switch (d) {
    case 64: return by_rt<64>(rt, grid, q, pa, pm, o, lse, p, s);
    case 128: return by_rt<128>(rt, grid, q, pa, pm, o, lse, p, s);
    case 256: return by_rt<256>(rt, grid, q, pa, pm, o, lse, p, s);
    case 512: return by_rt<512>(rt, grid, q, pa, pm, o, lse, p, s);
    default: return hipErrorInvalidValue;
    }
}

template <int D, int RT>
static int occ_of()
{
    if constexpr (!has_instance<D>()) {
        return 0;
    } else if constexpr (slices_of<D>() > 1) {
        constexpr int DS = slices_of<D>();
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, rkv_split_kernel<RKV_KT, RKV_VT, 128, RT, DS>,
                                                         64 * Shape<RKV_KT, RKV_VT, 128>::waves(sp_rows(RT, DS)), 0) !=
            hipSuccess) {
            (void)hipGetLastError();
            return 0;
        }
        return n;
    } else {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, rkv_split_kernel<RKV_KT, RKV_VT, D, RT>,
                                                         64 * Shape<RKV_KT, RKV_VT, D>::waves(RT), 0) != hipSuccess) {
            (void)hipGetLastError();
            return 0;
        }
        return n;
    }
}

template <int D>
static int occ_by_rt(int rt)
{
    switch (rt) {
    case 1: return occ_of<D, 1>();
    case 2: return occ_of<D, 2>();
    case 4: return occ_of<D, 4>();
    case 5: return occ_of<D, 5>();
    case 8: return occ_of<D, 8>();
    case 16: return occ_of<D, 16>();
    default: return 0;
    }
}

#define RKV_NAME_OCC(kt, vt) RKV_CAT4(split_occupancy_k, kt, _v, vt)
// Workgroups of this instance that fit one compute unit (0 if unknown).
int RKV_NAME_OCC(RKV_KT, RKV_VT)(int d, int rt)
{
    switch (d) {
    case 64: return occ_by_rt<64>(rt);
    case 128: return occ_by_rt<128>(rt);
    case 256: return occ_by_rt<256>(rt);
    case 512: return occ_by_rt<512>(rt);
    default: return 0;
    }
}

template <int D>
static int nw_by_rt(int rt)
{
    constexpr int DS = slices_of<D>();
    using Sh = Shape<RKV_KT, RKV_VT, (DS > 1 ? 128 : D)>;
    if (!has_instance<D>()) return 0;
    switch (rt) {
    case 1: return Sh::waves(sp_rows(1, DS));
    case 2: return Sh::waves(sp_rows(2, DS));
    case 4: return Sh::waves(sp_rows(4, DS));
    case 5: return Sh::waves(sp_rows(5, DS));
    case 8: return Sh::waves(sp_rows(8, DS));
    case 16: return Sh::waves(sp_rows(16, DS));
    default: return 0;
    }
}

#define RKV_NAME_NW(kt, vt) RKV_CAT4(split_waves_k, kt, _v, vt)
// Waves per workgroup of an instance.
int RKV_NAME_NW(RKV_KT, RKV_VT)(int d, int rt)
{
    switch (d) {
    case 64: return nw_by_rt<64>(rt);
    case 128: return nw_by_rt<128>(rt);
    case 256: return nw_by_rt<256>(rt);
    case 512: return nw_by_rt<512>(rt);
    default: return 0;
    }
}

// The shared-decode kernel (attend_shd.h): block-type K, q4_0 V, head_dim
// 128, 16 rows per wave, 4 row groups and 2 KV heads per workgroup; absent
// (invalid value / occupancy 0) for the other type pairs.
#define RKV_NAME_SHD(kt, vt) RKV_CAT4(launch_split_shd_k, kt, _v, vt)
hipError_t RKV_NAME_SHD(RKV_KT, RKV_VT)(dim3 grid, const float *q, float *pa, float2 *pm, float *o, float *lse,
                                        const SplitParams &p, hipStream_t s)
{
    if constexpr (ShdShape<RKV_KT, RKV_VT>::OK) {
        hipLaunchKernelGGL((rkv_split_shd_kernel<RKV_KT, RKV_VT>), grid, dim3(64 * kShdWaves), 0, s, q, pa, pm, o, lse,
                           p);
        return hipGetLastError();
    } else {
        return hipErrorInvalidValue;
    }
}

#define RKV_NAME_SHD_OCC(kt, vt) RKV_CAT4(split_shd_occupancy_k, kt, _v, vt)
int RKV_NAME_SHD_OCC(RKV_KT, RKV_VT)()
{
    if constexpr (ShdShape<RKV_KT, RKV_VT>::OK) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, rkv_split_shd_kernel<RKV_KT, RKV_VT>, 64 * kShdWaves, 0) !=
            hipSuccess) {
            (void)hipGetLastError();
            return 0;
        }
        return n;
    } else {
        return 0;
    }
}

#define RKV_NAME_SHD_OK(kt, vt) RKV_CAT4(split_shd_supported_k, kt, _v, vt)
bool RKV_NAME_SHD_OK(RKV_KT, RKV_VT)() { return ShdShape<RKV_KT, RKV_VT>::OK; }


// The staged-tile kernel for many rows per KV head (attend_rgs.h): f16 K and
// V at head_dim 128, built with the f16 / f16 pair only.
#if RKV_KT == 1 && RKV_VT == 1
hipError_t launch_split_rgs(dim3 grid, const float *q, float *pa, float2 *pm, float *o, float *lse,
                            const SplitParams &p, hipStream_t s)
{
    hipLaunchKernelGGL(rkv_split_rgs_kernel, grid, dim3(64 * kRgsRG), 0, s, q, pa, pm, o, lse, p);
    return hipGetLastError();
}

int split_rgs_occupancy()
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, rkv_split_rgs_kernel, 64 * kRgsRG, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return n;
}
#endif

}  // namespace rkv
