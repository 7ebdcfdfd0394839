// Matrix-core decode, host side: which shapes have a compiled kernel, how many
// blocks of it a CU holds, and the launch of the decode kernel for the head_dim
// (the caller then launches the split combine).
#include <math.h>

#include "decode_fast.h"

namespace aqkv {
namespace {

// compiled (d, w, m / 64) shapes of decode_fast_kernel, see decode_fast_d*.hip
bool fast_shape(int d, int w, int mc) {
  if (w >= 1 && w <= 3) return mc == d / 64;
  if (w != 0) return false;
  switch (d) {
    case 64: return mc >= 1 && mc <= 4;
    case 128: return mc == 1 || mc == 2 || mc == 3 || mc == 4 || mc == 6 || mc == 8;
    case 256: return mc == 2 || mc == 4 || mc == 6 || mc == 8;
    default: return false;
  }
}

}  // namespace

bool decode_mfma_supported(int d, int w, int g, int m, int vb, bool sf) {
  if (g != 1 && g != 2 && g != 4 && g != 8) return false;
  if (vb != 2 && vb != 4) return false;
  if (m % 64 || !fast_shape(d, w, m / 64)) return false;
  return fast::smem_of(d, w, m / 64, g, vb, sf) <= 160 * 1024;
}

int decode_mfma_blocks_per_cu(int d, int w, int g, int m, int vb, bool sf) {
  const int smem = fast::smem_of(d, w, m / 64, g, vb, sf);
  int by_lds = (160 * 1024) / smem;
  const int by_regs = fast::waves_per_simd(d, g);   // blocks of 4 waves = waves per SIMD
  if (by_lds > by_regs) by_lds = by_regs;
  return by_lds < 1 ? 1 : by_lds;
}

hipError_t launch_decode_mfma(const DecodeJob &job, hipStream_t stream) {
  switch (job.d) {
    case 64: return launch_decode_fast_d64(job, stream);
    case 128: return launch_decode_fast_d128(job, stream);
    default: return launch_decode_fast_d256(job, stream);
  }
}

}  // namespace aqkv
