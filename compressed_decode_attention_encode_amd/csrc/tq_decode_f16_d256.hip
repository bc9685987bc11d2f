// Compiled instantiations of the decode kernel: 16-bit keys (V-only mode), head_dim 256, n_rep
// 1..8, group-32 symmetric 2/4-bit values and rotated Lloyd-Max 2/3/4-bit values, on the matrix
// cores with 32-token wave tiles (a 64-token tile of 512-byte key rows does not fit a group's LDS
// share); fp16 rows use the fp16 products, bf16 rows the bf16 ones (the storage type is the
// layout's input type, chosen at run time).
#include "tq_decode_mma.h"

namespace tq {

namespace {
template <int VK, int VB>
MainKernel pick(int nrep) {
  switch (nrep) {
    case 1: return mma_kernel_kv<256, 1, TQ_K_F16, 16, VK, VB, 32>();
    case 2: return mma_kernel_kv<256, 2, TQ_K_F16, 16, VK, VB, 32>();
    case 3: return mma_kernel_kv<256, 3, TQ_K_F16, 16, VK, VB, 32>();
    case 4: return mma_kernel_kv<256, 4, TQ_K_F16, 16, VK, VB, 32>();
    case 5: return mma_kernel_kv<256, 5, TQ_K_F16, 16, VK, VB, 32>();
    case 6: return mma_kernel_kv<256, 6, TQ_K_F16, 16, VK, VB, 32>();
    case 7: return mma_kernel_kv<256, 7, TQ_K_F16, 16, VK, VB, 32>();
    case 8: return mma_kernel_kv<256, 8, TQ_K_F16, 16, VK, VB, 32>();
    default: return MainKernel{nullptr, nullptr};
  }
}
}  // namespace

MainKernel find_mma_f16_d256(int nrep, int vk, int vb) {
  if (vk == TQ_V_GROUP_SYM && vb == 2) return pick<TQ_V_GROUP_SYM, 2>(nrep);
  if (vk == TQ_V_GROUP_SYM && vb == 4) return pick<TQ_V_GROUP_SYM, 4>(nrep);
  if (vk == TQ_V_LM_ROT && vb == 2) return pick<TQ_V_LM_ROT, 2>(nrep);
  if (vk == TQ_V_LM_ROT && vb == 3) return pick<TQ_V_LM_ROT, 3>(nrep);
  if (vk == TQ_V_LM_ROT && vb == 4) return pick<TQ_V_LM_ROT, 4>(nrep);
  return MainKernel{nullptr, nullptr};
}

}  // namespace tq
