// affine_scan.hip -- scan of affine maps h -> a h + b along rows, with the
// wave-wide associative scan of device_common.hpp.
//
// Each step of the selective SSM's recurrence is such a map (reading guide of
// arXiv 2312.00752, "Yöntem": the discrete state is the previous state times
// the discretised A plus the discretised input), and the maps compose
// associatively, which is what lets a scan run in parallel over time (the
// parallel prefix scan of the mamba-minimal page's Hacker News comments).  The
// library uses the same primitive to fold the segments of a split sequence;
// this kernel exposes it on plain arrays (for example to fold the segment
// aggregates of a sequence sharded over several devices).
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssm {

// One wave per row.  A row is taken 64 positions at a time: lanes load the
// pairs of their positions (the identity past the end), the wave scans them,
// every lane applies the composed map to the state carried in from the
// previous piece, and lane 63 (the last position, since identities follow it)
// carries the state on.
__global__ void __launch_bounds__(256) affine_scan_kernel(AffineScanArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;  // uniform over the wave: whole waves leave
  const float *ar = a.a + row * a.len, *br = a.b + row * a.len;
  float *hr = a.h + row * a.len;
  float carry = a.h0 ? a.h0[row] : 0.0f;
  for (int64_t p0 = 0; p0 < a.len; p0 += 64) {
    const int64_t k = p0 + lane;                            // position in scan order
    const bool valid = k < a.len;
    const int64_t i = a.reverse ? a.len - 1 - k : k;        // element
    float x = valid ? ar[i] : 1.0f, y = valid ? br[i] : 0.0f;
    wave_affine_scan(x, y);
    const float s = fmaf(x, carry, y);
    if (valid) hr[i] = s;
    carry = __shfl(s, 63, 64);
  }
}

hipError_t launch_affine_scan(const AffineScanArgs &a, hipStream_t s) {
  const int64_t blocks = (a.rows + 3) / 4;
  hipLaunchKernelGGL(affine_scan_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ssm
