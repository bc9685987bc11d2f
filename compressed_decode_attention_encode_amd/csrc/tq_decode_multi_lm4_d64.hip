// Compiled instantiations of the multi-query decode kernel (several consecutive queries per
// step against one pass over the packed cache) for 4-bit Lloyd-Max + QJL keys, head_dim 64,
// group-32 symmetric 2/4-bit values: n_rep 1..8 with 2 queries, n_rep 1, 2, 4 with 4 queries, n_rep 1, 2
// with 8 queries (n_query x n_rep <= 16).
#include "tq_decode_mma.h"

namespace tq {

namespace {
template <int VB>
MainKernel pick(int nrep, int nq) {
  if (nq == 2) {
    switch (nrep) {
      case 1: return mma_kernel<64, 1, 4, VB, 2>();
      case 2: return mma_kernel<64, 2, 4, VB, 2>();
      case 3: return mma_kernel<64, 3, 4, VB, 2>();
      case 4: return mma_kernel<64, 4, 4, VB, 2>();
      case 5: return mma_kernel<64, 5, 4, VB, 2>();
      case 6: return mma_kernel<64, 6, 4, VB, 2>();
      case 7: return mma_kernel<64, 7, 4, VB, 2>();
      case 8: return mma_kernel<64, 8, 4, VB, 2>();
      default: break;
    }
  } else if (nq == 4) {
    if (nrep == 1) return mma_kernel<64, 1, 4, VB, 4>();
    if (nrep == 2) return mma_kernel<64, 2, 4, VB, 4>();
    if (nrep == 4) return mma_kernel<64, 4, 4, VB, 4>();
  } else if (nq == 8) {
    if (nrep == 1) return mma_kernel<64, 1, 4, VB, 8>();
    if (nrep == 2) return mma_kernel<64, 2, 4, VB, 8>();
  }
  return MainKernel{nullptr, nullptr};
}
}  // namespace

MainKernel find_multi_lm4_d64(int nrep, int nq, int vb) {
  if (vb == 2) return pick<2>(nrep, nq);
  if (vb == 4) return pick<4>(nrep, nq);
  return MainKernel{nullptr, nullptr};
}

}  // namespace tq
