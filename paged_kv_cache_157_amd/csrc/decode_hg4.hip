// decode_hg4.hip -- instantiates the head-group decode kernel with groups of
// four KV heads, for every (cache dtype, head_dim, G >= 2) the library
// serves; a translation unit of its own so it compiles beside decode.hip.
#include <type_traits>

#include "decode_hg.h"

namespace pa {

DecodeKernels decode_hg4_kernels(int cache_dtype, int head_dim, int group)
{
    constexpr int HPG = 4;
    auto pick = [](auto kern) { return DecodeKernels{(const void *)kern, 64 * HPG}; };
    auto by_g = [&](auto cdt, auto dh) -> DecodeKernels {
        constexpr int CDT = decltype(cdt)::value, D = decltype(dh)::value;
        switch (group) {
        case 2: return pick(hg::decode_hg_kernel<CDT, D, 2, HPG>);
        case 3: return pick(hg::decode_hg_kernel<CDT, D, 3, HPG>);
        case 4: return pick(hg::decode_hg_kernel<CDT, D, 4, HPG>);
        case 5: return pick(hg::decode_hg_kernel<CDT, D, 5, HPG>);
        case 6: return pick(hg::decode_hg_kernel<CDT, D, 6, HPG>);
        case 7: return pick(hg::decode_hg_kernel<CDT, D, 7, HPG>);
        default: return pick(hg::decode_hg_kernel<CDT, D, 8, HPG>);
        }
    };
    using DF32 = std::integral_constant<int, DT_F32>;
    using DBF16 = std::integral_constant<int, DT_BF16>;
    using DFP8 = std::integral_constant<int, DT_FP8>;
    using D64 = std::integral_constant<int, 64>;
    using D128 = std::integral_constant<int, 128>;
    if (cache_dtype == DT_F32)
        return by_g(DF32{}, D64{});
    if (cache_dtype == DT_BF16)
        return head_dim == 64 ? by_g(DBF16{}, D64{}) : by_g(DBF16{}, D128{});
    if (head_dim == 64) {
        switch (group) {
        case 2: return pick(hg::decode_hg_kernel<DT_FP8, 64, 2, HPG>);
        case 3: return pick(hg::decode_hg_kernel<DT_FP8, 64, 3, HPG>);
        default: return pick(hg::decode_hg_kernel<DT_FP8, 64, 4, HPG>);
        }
    }
    return by_g(DFP8{}, D128{});
}

}  // namespace pa
