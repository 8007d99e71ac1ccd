// qg_kquant.hip -- the dense GEMV kernels for the K-quant super-block
// formats Q4_K and Q6_K (the GGUF formats of the imp engine's models: imp
// README, "Features" table, Quantization row; imp release notes v0.7.0,
// Q4_K_M).  Activations are staged in fp32 for both x types (each weight is
// formed in fp32 before its product, so the bf16 dot path does not apply);
// one token runs the one-batch kernel when a wave's stream is at most 8
// steps, as Q8_0 does.
#include "qg_common.h"

namespace qg {

// Q6_K with bf16 x runs the bf16 dot path (its q - 32 is exact in bf16);
// Q4_K forms each weight in fp32 and stages fp32 activations.
template <int FMT>
static dense_fn dense_for(int xt, int m)
{
    constexpr bool DOT = FMT == QG_Q6_K;
    return xt == QG_BF16 ? pick_dense<FMT, true, DOT>(m) : pick_dense<FMT, false, false>(m);
}

template <int FMT>
static dense_fn dense_one_for(int xt, int m, int u)
{
    constexpr bool DOT = FMT == QG_Q6_K;
    return xt == QG_BF16 ? pick_dense_one<FMT, true, DOT>(m, u) : pick_dense_one<FMT, false, false>(m, u);
}

dense_fn dense_kernel_kq(int fmt, int xt, int m)
{
    return fmt == QG_Q4_K ? dense_for<QG_Q4_K>(xt, m) : dense_for<QG_Q6_K>(xt, m);
}

dense_fn dense_one_kernel_kq(int fmt, int xt, int m, int u)
{
    return fmt == QG_Q4_K ? dense_one_for<QG_Q4_K>(xt, m, u) : dense_one_for<QG_Q6_K>(xt, m, u);
}

} // namespace qg
