// Compiled instantiations of the decode kernel for 3-bit Lloyd-Max + QJL keys, head_dim 64,
// n_rep 1..8, group-32 symmetric or min/max 2/4-bit values (min/max: matrix cores at every n_rep); n_rep 1 and 2 on the vector ALUs (per-token
// work grows with n_rep there and is still small), n_rep 3..8 on the matrix cores.
#include "tq_decode_mma.h"

namespace tq {

namespace {
template <int VB>
MainKernel pick(int nrep) {
  switch (nrep) {
    case 1: return main_kernel<64, 1, TQ_K_LM_QJL, 3, TQ_V_GROUP_SYM, VB>();
    case 2: return main_kernel<64, 2, TQ_K_LM_QJL, 3, TQ_V_GROUP_SYM, VB>();
    case 3: return mma_kernel<64, 3, 3, VB>();
    case 4: return mma_kernel<64, 4, 3, VB>();
    case 5: return mma_kernel<64, 5, 3, VB>();
    case 6: return mma_kernel<64, 6, 3, VB>();
    case 7: return mma_kernel<64, 7, 3, VB>();
    case 8: return mma_kernel<64, 8, 3, VB>();
    default: return MainKernel{nullptr, nullptr};
  }
}
}  // namespace

// group-32 min/max values: the matrix-core kernel at every n_rep
template <int VB>
MainKernel pick_minmax(int nrep) {
  constexpr int KK = TQ_K_LM_QJL, VK = TQ_V_GROUP_ASYM;
  switch (nrep) {
    case 1: return mma_kernel_kv<64, 1, KK, 3, VK, VB>();
    case 2: return mma_kernel_kv<64, 2, KK, 3, VK, VB>();
    case 3: return mma_kernel_kv<64, 3, KK, 3, VK, VB>();
    case 4: return mma_kernel_kv<64, 4, KK, 3, VK, VB>();
    case 5: return mma_kernel_kv<64, 5, KK, 3, VK, VB>();
    case 6: return mma_kernel_kv<64, 6, KK, 3, VK, VB>();
    case 7: return mma_kernel_kv<64, 7, KK, 3, VK, VB>();
    case 8: return mma_kernel_kv<64, 8, KK, 3, VK, VB>();
    default: return MainKernel{nullptr, nullptr};
  }
}

MainKernel find_main_lm3_d64(int nrep, int vk, int vb) {
  if (vk == TQ_V_GROUP_SYM && vb == 2) return pick<2>(nrep);
  if (vk == TQ_V_GROUP_SYM && vb == 4) return pick<4>(nrep);
  if (vk == TQ_V_GROUP_ASYM && vb == 2) return pick_minmax<2>(nrep);
  if (vk == TQ_V_GROUP_ASYM && vb == 4) return pick_minmax<4>(nrep);
  return MainKernel{nullptr, nullptr};
}

}  // namespace tq
