// Compiled instantiations of the decode kernels: 16-bit keys (V-only mode), head_dim 64, n_rep
// 1..8, group-32 symmetric 2/4-bit values and rotated Lloyd-Max 2/3/4-bit values; fp16 keys at
// n_rep 3..8 also on the matrix cores (the stored rows are exact fp16 operands).
#include "tq_decode_mma.h"

namespace tq {

namespace {
template <int KK, int KB, int VK, int VB>
MainKernel pick(int nrep) {
  switch (nrep) {
    case 1: return main_kernel<64, 1, KK, KB, VK, VB>();
    case 2: return main_kernel<64, 2, KK, KB, VK, VB>();
    case 3: return main_kernel<64, 3, KK, KB, VK, VB>();
    case 4: return main_kernel<64, 4, KK, KB, VK, VB>();
    case 5: return main_kernel<64, 5, KK, KB, VK, VB>();
    case 6: return main_kernel<64, 6, KK, KB, VK, VB>();
    case 7: return main_kernel<64, 7, KK, KB, VK, VB>();
    case 8: return main_kernel<64, 8, KK, KB, VK, VB>();
    default: return MainKernel{nullptr, nullptr};
  }
}
template <int VK, int VB>
MainKernel pick_mma(int nrep) {
  switch (nrep) {
    case 3: return mma_kernel_kv<64, 3, TQ_K_F16, 16, VK, VB>();
    case 4: return mma_kernel_kv<64, 4, TQ_K_F16, 16, VK, VB>();
    case 5: return mma_kernel_kv<64, 5, TQ_K_F16, 16, VK, VB>();
    case 6: return mma_kernel_kv<64, 6, TQ_K_F16, 16, VK, VB>();
    case 7: return mma_kernel_kv<64, 7, TQ_K_F16, 16, VK, VB>();
    case 8: return mma_kernel_kv<64, 8, TQ_K_F16, 16, VK, VB>();
    default: return MainKernel{nullptr, nullptr};
  }
}
}  // namespace

MainKernel find_mma_f16_d64(int nrep, int vk, int vb) {
  if (vk == TQ_V_GROUP_SYM && vb == 2) return pick_mma<TQ_V_GROUP_SYM, 2>(nrep);
  if (vk == TQ_V_GROUP_SYM && vb == 4) return pick_mma<TQ_V_GROUP_SYM, 4>(nrep);
  if (vk == TQ_V_LM_ROT && vb == 2) return pick_mma<TQ_V_LM_ROT, 2>(nrep);
  if (vk == TQ_V_LM_ROT && vb == 3) return pick_mma<TQ_V_LM_ROT, 3>(nrep);
  if (vk == TQ_V_LM_ROT && vb == 4) return pick_mma<TQ_V_LM_ROT, 4>(nrep);
  return MainKernel{nullptr, nullptr};
}

MainKernel find_main_f16_d64(int nrep, int vk, int vb) {
  if (vk == TQ_V_GROUP_SYM && vb == 2) return pick<TQ_K_F16, 16, TQ_V_GROUP_SYM, 2>(nrep);
  if (vk == TQ_V_GROUP_SYM && vb == 4) return pick<TQ_K_F16, 16, TQ_V_GROUP_SYM, 4>(nrep);
  if (vk == TQ_V_LM_ROT && vb == 2) return pick<TQ_K_F16, 16, TQ_V_LM_ROT, 2>(nrep);
  if (vk == TQ_V_LM_ROT && vb == 3) return pick<TQ_K_F16, 16, TQ_V_LM_ROT, 3>(nrep);
  if (vk == TQ_V_LM_ROT && vb == 4) return pick<TQ_K_F16, 16, TQ_V_LM_ROT, 4>(nrep);
  return MainKernel{nullptr, nullptr};
}

}  // namespace tq
