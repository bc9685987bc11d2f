// Compiled instantiations of the decode kernel: per-block affine 2-bit keys (vllm-metal guide,
// compression-ratio table), head_dim 64, n_rep 1..8, rotated Lloyd-Max 2/3/4-bit values, all on
// the matrix cores (the query rows beyond n_rep are zero operand columns).
#include "tq_decode_mma.h"

namespace tq {

namespace {
template <int VB>
MainKernel pick(int nrep) {
  constexpr int KK = TQ_K_AFFINE8, VK = TQ_V_LM_ROT;
  switch (nrep) {
    case 1: return mma_kernel_kv<64, 1, KK, 2, VK, VB>();
    case 2: return mma_kernel_kv<64, 2, KK, 2, VK, VB>();
    case 3: return mma_kernel_kv<64, 3, KK, 2, VK, VB>();
    case 4: return mma_kernel_kv<64, 4, KK, 2, VK, VB>();
    case 5: return mma_kernel_kv<64, 5, KK, 2, VK, VB>();
    case 6: return mma_kernel_kv<64, 6, KK, 2, VK, VB>();
    case 7: return mma_kernel_kv<64, 7, KK, 2, VK, VB>();
    case 8: return mma_kernel_kv<64, 8, KK, 2, VK, VB>();
    default: return MainKernel{nullptr, nullptr};
  }
}
}  // namespace

MainKernel find_main_aff2_d64(int nrep, int vk, int vb) {
  if (vk != TQ_V_LM_ROT) return MainKernel{nullptr, nullptr};
  switch (vb) {
    case 2: return pick<2>(nrep);
    case 3: return pick<3>(nrep);
    case 4: return pick<4>(nrep);
    default: return MainKernel{nullptr, nullptr};
  }
}

}  // namespace tq
