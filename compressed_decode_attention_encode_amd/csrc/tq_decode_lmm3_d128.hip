// Compiled instantiations of the decode main kernel: MSE-only 3-bit Lloyd-Max keys (no QJL
// term), head_dim 128, n_rep 1..8, group-32 symmetric 2/4-bit values and rotated Lloyd-Max
// 2/3/4-bit values (group values at n_rep 3..8 on the matrix cores).
#include "tq_decode_mma.h"

namespace tq {

namespace {
// group values at n_rep 3..8: the matrix-core kernel (codebook term only)
template <int VB>
MainKernel pick_mma(int nrep) {
  constexpr int KK = TQ_K_LM_MSE, VK = TQ_V_GROUP_SYM;
  switch (nrep) {
    case 3: return mma_kernel_kv<128, 3, KK, 3, VK, VB>();
    case 4: return mma_kernel_kv<128, 4, KK, 3, VK, VB>();
    case 5: return mma_kernel_kv<128, 5, KK, 3, VK, VB>();
    case 6: return mma_kernel_kv<128, 6, KK, 3, VK, VB>();
    case 7: return mma_kernel_kv<128, 7, KK, 3, VK, VB>();
    case 8: return mma_kernel_kv<128, 8, KK, 3, VK, VB>();
    default: return MainKernel{nullptr, nullptr};
  }
}

template <int KK, int KB, int VK, int VB>
MainKernel pick(int nrep) {
  switch (nrep) {
    case 1: return main_kernel<128, 1, KK, KB, VK, VB>();
    case 2: return main_kernel<128, 2, KK, KB, VK, VB>();
    case 3: return main_kernel<128, 3, KK, KB, VK, VB>();
    case 4: return main_kernel<128, 4, KK, KB, VK, VB>();
    case 5: return main_kernel<128, 5, KK, KB, VK, VB>();
    case 6: return main_kernel<128, 6, KK, KB, VK, VB>();
    case 7: return main_kernel<128, 7, KK, KB, VK, VB>();
    case 8: return main_kernel<128, 8, KK, KB, VK, VB>();
    default: return MainKernel{nullptr, nullptr};
  }
}
}  // namespace

MainKernel find_main_lmm3_d128(int nrep, int vk, int vb) {
  if (vk == TQ_V_GROUP_SYM && vb == 2) return nrep >= 3 ? pick_mma<2>(nrep) : pick<TQ_K_LM_MSE, 3, TQ_V_GROUP_SYM, 2>(nrep);
  if (vk == TQ_V_GROUP_SYM && vb == 4) return nrep >= 3 ? pick_mma<4>(nrep) : pick<TQ_K_LM_MSE, 3, TQ_V_GROUP_SYM, 4>(nrep);
  if (vk == TQ_V_LM_ROT && vb == 2) return pick<TQ_K_LM_MSE, 3, TQ_V_LM_ROT, 2>(nrep);
  if (vk == TQ_V_LM_ROT && vb == 3) return pick<TQ_K_LM_MSE, 3, TQ_V_LM_ROT, 3>(nrep);
  if (vk == TQ_V_LM_ROT && vb == 4) return pick<TQ_K_LM_MSE, 3, TQ_V_LM_ROT, 4>(nrep);
  return MainKernel{nullptr, nullptr};
}

}  // namespace tq
