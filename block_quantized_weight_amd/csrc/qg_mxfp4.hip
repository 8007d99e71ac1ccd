// qg_mxfp4.hip -- MXFP4 instantiations of the dense and expert GEMV kernels.
#include "qg_chain.h"
#include "qg_fused.h"
#include "qg_mfma.h"
#include "qg_moe_stream.h"

namespace qg {

dense_fn dense_kernel_mxfp4(int xt, int m)
{
    return xt == QG_BF16 ? pick_dense<QG_MXFP4, true, true>(m) : pick_dense<QG_MXFP4, false, false>(m);
}

dense_fn dense_one_kernel_mxfp4(int xt, int m, int u)
{
    return xt == QG_BF16 ? pick_dense_one<QG_MXFP4, true, true>(m, u) : pick_dense_one<QG_MXFP4, false, false>(m, u);
}

hipError_t launch_moe_mxfp4(int xt, int mode, const Plan &p, const MoeArgs &a, int maxdistinct, size_t lds,
                           const void *x, float *y, hipStream_t s)
{
    if (xt == QG_BF16) return launch_moe_t<QG_MXFP4, true, true>(mode, p, a, maxdistinct, lds, x, y, s);
    return launch_moe_t<QG_MXFP4, false, false>(mode, p, a, maxdistinct, lds, x, y, s);
}

const void *chain_kernel_mxfp4(int xt, int m)
{
    return xt == QG_BF16 ? pick_chain<QG_MXFP4, true, true>(m) : pick_chain<QG_MXFP4, false, false>(m);
}

int chain_error_mxfp4(bool clear) { return chain_error_read(clear); }

mfma_fn mfma_kernel_mxfp4(int L, int tg, int nw) { return pick_mfma<QG_MXFP4>(L, tg, nw); }

moe_stream_fn moe_stream_kernel_mxfp4(int xt, int mode, int ms, bool norm, bool glu, bool short_items,
                                     bool wide)
{
    return xt == QG_BF16 ? pick_moe_stream<QG_MXFP4, true, true>(mode, ms, norm, glu, short_items, wide)
                         : pick_moe_stream<QG_MXFP4, false, false>(mode, ms, norm, glu, short_items, wide);
}

dense_ep_fn dense_one_ep_kernel_mxfp4(int xt, int m, int u) { return pick_dense_one_ep<QG_MXFP4>(xt, m, u); }

dense_ep_fn dense_ep_kernel_mxfp4(int xt, int m, bool norm, int glu)
{
    return pick_dense_ep_fmt<QG_MXFP4>(xt, m, norm, glu);
}

} // namespace qg
