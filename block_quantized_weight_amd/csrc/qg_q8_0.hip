// qg_q8_0.hip -- Q8_0 instantiations of the dense and expert GEMV kernels.
#include "qg_chain.h"
#include "qg_fused.h"
#include "qg_mfma.h"
#include "qg_moe_stream.h"

namespace qg {

dense_fn dense_kernel_q8_0(int xt, int m)
{
    return xt == QG_BF16 ? pick_dense<QG_Q8_0, true, false>(m) : pick_dense<QG_Q8_0, false, false>(m);
}

dense_fn dense_one_kernel_q8_0(int xt, int m, int u)
{
    return xt == QG_BF16 ? pick_dense_one<QG_Q8_0, true, false>(m, u) : pick_dense_one<QG_Q8_0, false, false>(m, u);
}

hipError_t launch_moe_q8_0(int xt, int mode, const Plan &p, const MoeArgs &a, int maxdistinct, size_t lds,
                           const void *x, float *y, hipStream_t s)
{
    if (xt == QG_BF16) return launch_moe_t<QG_Q8_0, true, false>(mode, p, a, maxdistinct, lds, x, y, s);
    return launch_moe_t<QG_Q8_0, false, false>(mode, p, a, maxdistinct, lds, x, y, s);
}

const void *chain_kernel_q8_0(int xt, int m)
{
    return xt == QG_BF16 ? pick_chain<QG_Q8_0, true, false>(m) : pick_chain<QG_Q8_0, false, false>(m);
}

int chain_error_q8_0(bool clear) { return chain_error_read(clear); }

mfma_fn mfma_kernel_q8_0(int L, int tg) { return pick_mfma<QG_Q8_0>(L, tg); }

moe_stream_fn moe_stream_kernel_q8_0(int xt, int mode, int ms, bool norm, bool glu)
{
    return xt == QG_BF16 ? pick_moe_stream<QG_Q8_0, true, false>(mode, ms, norm, glu)
                         : pick_moe_stream<QG_Q8_0, false, false>(mode, ms, norm, glu);
}

dense_ep_fn dense_one_ep_kernel_q8_0(int xt, int m, int u) { return pick_dense_one_ep<QG_Q8_0>(xt, m, u); }

dense_ep_fn dense_ep_kernel_q8_0(int xt, int m, bool norm, int glu)
{
    return pick_dense_ep_fmt<QG_Q8_0>(xt, m, norm, glu);
}

} // namespace qg
