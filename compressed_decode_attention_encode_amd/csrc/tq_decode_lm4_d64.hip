// Compiled instantiations of the decode kernel for 4-bit Lloyd-Max + QJL keys, head_dim 64,
// n_rep 1..8, group-32 symmetric 2/4-bit values: n_rep 1 and 2 on the vector ALUs (per-token
// work grows with n_rep there and is still small), n_rep 3..8 on the matrix cores.
#include "tq_decode_mma.h"

namespace tq {

namespace {
template <int VB>
MainKernel pick(int nrep) {
  switch (nrep) {
    case 1: return main_kernel<64, 1, TQ_K_LM_QJL, 4, TQ_V_GROUP_SYM, VB>();
    case 2: return main_kernel<64, 2, TQ_K_LM_QJL, 4, TQ_V_GROUP_SYM, VB>();
    case 3: return mma_kernel<64, 3, 4, VB>();
    case 4: return mma_kernel<64, 4, 4, VB>();
    case 5: return mma_kernel<64, 5, 4, VB>();
    case 6: return mma_kernel<64, 6, 4, VB>();
    case 7: return mma_kernel<64, 7, 4, VB>();
    case 8: return mma_kernel<64, 8, 4, VB>();
    default: return MainKernel{nullptr, nullptr};
  }
}
}  // namespace

MainKernel find_main_lm4_d64(int nrep, int vk, int vb) {
  if (vk == TQ_V_GROUP_SYM && vb == 2) return pick<2>(nrep);
  if (vk == TQ_V_GROUP_SYM && vb == 4) return pick<4>(nrep);
  return MainKernel{nullptr, nullptr};
}

}  // namespace tq
