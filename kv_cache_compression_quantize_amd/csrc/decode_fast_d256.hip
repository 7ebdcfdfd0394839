// Matrix-core decode kernels for head_dim 256 (template in decode_fast.h; the
// compiled sketch sizes are the ones decode_mfma_supported accepts).
#include "decode_fast.h"

namespace aqkv {

hipError_t launch_decode_fast_d256(const DecodeJob &job, hipStream_t stream) {
  using namespace fast;
  switch (job.w) {
    case 1: return launch_fast_m<256, 1, 4>(job, stream);
    case 2: return launch_fast_m<256, 2, 4>(job, stream);
    case 3: return launch_fast_m<256, 3, 4>(job, stream);
    default:
      switch (job.m / 64) {
      case 2: return launch_fast_m<256, 0, 2>(job, stream);
      case 4: return launch_fast_m<256, 0, 4>(job, stream);
      case 6: return launch_fast_m<256, 0, 6>(job, stream);
      default: return launch_fast_m<256, 0, 8>(job, stream);
      }
  }
}

}  // namespace aqkv
