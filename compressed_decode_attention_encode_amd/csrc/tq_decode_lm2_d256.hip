// Compiled instantiations of the decode kernel: 2-bit Lloyd-Max + QJL keys, head_dim 256,
// n_rep 1..8, group-32 symmetric 2/4-bit values: n_rep 1 and 2 on the vector ALUs, n_rep 3..8
// on the matrix cores with 32-token wave tiles.
#include "tq_decode_mma.h"

namespace tq {

namespace {
template <int VB>
MainKernel pick(int nrep) {
  constexpr int KK = TQ_K_LM_QJL, VK = TQ_V_GROUP_SYM;
  switch (nrep) {
    case 1: return main_kernel<256, 1, KK, 2, VK, VB>();
    case 2: return main_kernel<256, 2, KK, 2, VK, VB>();
    case 3: return mma_kernel_kv<256, 3, KK, 2, VK, VB, 32>();
    case 4: return mma_kernel_kv<256, 4, KK, 2, VK, VB, 32>();
    case 5: return mma_kernel_kv<256, 5, KK, 2, VK, VB, 32>();
    case 6: return mma_kernel_kv<256, 6, KK, 2, VK, VB, 32>();
    case 7: return mma_kernel_kv<256, 7, KK, 2, VK, VB, 32>();
    case 8: return mma_kernel_kv<256, 8, KK, 2, VK, VB, 32>();
    default: return MainKernel{nullptr, nullptr};
  }
}
}  // namespace

MainKernel find_main_lm2_d256(int nrep, int vk, int vb) {
  if (vk == TQ_V_GROUP_SYM && vb == 2) return pick<2>(nrep);
  if (vk == TQ_V_GROUP_SYM && vb == 4) return pick<4>(nrep);
  return MainKernel{nullptr, nullptr};
}

}  // namespace tq
