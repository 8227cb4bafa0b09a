// math_probe.hip -- test-only HIP library: runs the decoder's float32
// numerics (exp, log1p, the quotient log1p starts from, logsumexp) from
// ctc_prefix_beam_amd/csrc/device_math.h on the GPU over ranges of inputs, so
// that tests can compare them bit for bit with the oracle's C versions of the
// same operation sequences.  It is built with the decoder's flags (no
// contraction, no packed fp32) and is not part of the decoder library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../ctc_prefix_beam_amd/csrc/device_math.h"

namespace {

// element i: the float with bit pattern first + i (ops 0..2) or the pair
// (a[i], b[i]) (op 3); grid-stride over n elements
__global__ __launch_bounds__(256) void probe_kernel(int op, uint32_t first, int64_t n,
                                                    const float* a, const float* b, float* out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float x = __uint_as_float(first + (uint32_t)i);
    float y;
    switch (op) {
      case 0: y = ctcpb::exp_m80_0(x); break;
      case 1: y = ctcpb::log1p_0_1(x); break;
      case 2: y = ctcpb::quot_x_2px(x); break;
      default: y = ctcpb::lse(a[i], b[i]); break;
    }
    out[i] = y;
  }
}

}  // namespace

// out (device float32 [n]); a, b (device float32 [n]) used by op 3 only.
// Returns 0, 1 on an invalid argument, 4 if the launch fails.
extern "C" int math_probe(int op, uint32_t first_bits, int64_t n, const float* a, const float* b,
                          float* out, void* stream) {
  if (op < 0 || op > 3 || n < 0 || !out || (op == 3 && (!a || !b))) return 1;
  if (n == 0) return 0;
  const int64_t blocks64 = (n + 255) / 256;
  const int blocks = (int)(blocks64 < 65536 ? blocks64 : 65536);
  hipLaunchKernelGGL(probe_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     op, first_bits, n, a, b, out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
