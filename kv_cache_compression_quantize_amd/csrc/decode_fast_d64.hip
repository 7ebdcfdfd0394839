// Matrix-core decode kernels for head_dim 64 (template in decode_fast.h; the
// compiled sketch sizes are the ones decode_mfma_supported accepts).
#include "decode_fast.h"

namespace aqkv {

hipError_t launch_decode_fast_d64(const DecodeJob &job, hipStream_t stream) {
  using namespace fast;
  switch (job.w) {
    case 1: return launch_fast_m<64, 1, 1>(job, stream);
    case 2: return launch_fast_m<64, 2, 1>(job, stream);
    case 3: return launch_fast_m<64, 3, 1>(job, stream);
    default:
      switch (job.m / 64) {
      case 1: return launch_fast_m<64, 0, 1>(job, stream);
      case 2: return launch_fast_m<64, 0, 2>(job, stream);
      case 3: return launch_fast_m<64, 0, 3>(job, stream);
      default: return launch_fast_m<64, 0, 4>(job, stream);
      }
  }
}

}  // namespace aqkv
