// Matrix-core decode kernels for head_dim 128 (template in decode_fast.h; the
// compiled sketch sizes are the ones decode_mfma_supported accepts).
#include "decode_fast.h"

namespace aqkv {

hipError_t launch_decode_fast_d128(const DecodeJob &job, hipStream_t stream) {
  using namespace fast;
  switch (job.w) {
    case 1: return launch_fast_m<128, 1, 2>(job, stream);
    case 2: return launch_fast_m<128, 2, 2>(job, stream);
    case 3: return launch_fast_m<128, 3, 2>(job, stream);
    default:
      switch (job.m / 64) {
      case 1: return launch_fast_m<128, 0, 1>(job, stream);
      case 2: return launch_fast_m<128, 0, 2>(job, stream);
      case 3: return launch_fast_m<128, 0, 3>(job, stream);
      case 4: return launch_fast_m<128, 0, 4>(job, stream);
      case 6: return launch_fast_m<128, 0, 6>(job, stream);
      default: return launch_fast_m<128, 0, 8>(job, stream);
      }
  }
}

}  // namespace aqkv
