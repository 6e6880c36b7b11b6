// gemm_plain.hip -- plain packed GEMM (runs already along the contraction),
// used by the naive comparison path.
#include "gemm_kernel.h"

namespace mq {

int plain_gemm_splits(long long Ma, long long Nb, long long nkb) {
  return splitk_slices(Ma, Nb, nkb, (Ma + Nb) * nkb * 32, 2, false);  // per-row scales
}

hipError_t launch_plain_gemm(int fa, int fb, const uint8_t* ac, const uint8_t* as, const uint8_t* bc,
                             const uint8_t* bs, int Ma, int Nb, int nkb, float* out, int splits,
                             hipStream_t st) {
  PlainProb p;
  p.ac = ac; p.as = as; p.bc = bc; p.bs = bs; p.out = out; p.Ma = Ma; p.Nb = Nb; p.nkb = nkb;
  p.aRB = (int)run_bytes(fa); p.bRB = (int)run_bytes(fb);
  p.arb = nkb * p.aRB; p.brb = nkb * p.bRB;
  p.ac_bytes = (long long)Ma * p.arb; p.as_bytes = (long long)Ma * nkb;
  p.bc_bytes = (long long)Nb * p.brb; p.bs_bytes = (long long)Nb * nkb;
  p.pairs_per_split = ceil_div((nkb + 1) / 2, splits);
  return launch_tiled(fa, fb, p, Ma, Nb, splits, st);
}


}  // namespace mq
