// Segment scan of the sequence split of the GLA forward.
//
// A long sequence is cut into segments whose states are found in parallel.
// The recurrence of the page "Gated Linear Attention (GLA): Mathematical
// Foundations ...", section "The Gated Recurrent Update", is linear in the
// state and diagonal in its transition, so over one segment
//     S_end = diag(a) S_start + S_zero,
// with a = exp(sum of the segment's log-gates) per key channel and S_zero the
// state the segment reaches from S = 0 (the segment state pass computes both).
// This kernel runs that recurrence over the segments of each (sequence, head):
// it replaces each S_zero by the segment's incoming state S_start, in place,
// and writes the state after the last segment as the final state.
//
// The backward pass uses the same scan in the other direction: the gradient of
// the state obeys B_start = diag(a) B_end + B_zero over a segment (B_zero from
// the segment's own outputs), so with `reverse` the segments are visited from
// last to first, starting from the gradient of the final state, and each slot
// receives the gradient entering its segment from the later ones.
//
// One thread owns 4 consecutive elements of the d_k x d_v state for every
// segment of its unit; elements are independent, so 256 threads x (d_k d_v /
// 1024) workgroups per unit stream the states with 16-byte accesses.
#include "gla_device.h"
#include "gla_kernels.h"

namespace gla {

__global__ __launch_bounds__(256) void seg_scan_kernel(SegScanParams prm) {
  const int per = prm.dk * prm.dv / 1024;           // workgroups per unit
  const int unit = blockIdx.x / per;
  const int e = (blockIdx.x - unit * per) * 1024 + threadIdx.x * 4;
  const int row = e / prm.dv;                       // key channel of the 4 elements
  const long dkdv = (long)prm.dk * prm.dv;
  float4 S = prm.s0 ? *reinterpret_cast<const float4*>(prm.s0 + unit * dkdv + e)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < prm.nseg; ++k) {
    const int sgi = prm.reverse ? prm.nseg - 1 - k : k;
    const long it = (long)unit * prm.nseg + sgi;
    float4* slot = reinterpret_cast<float4*>(prm.seg_state + it * dkdv + e);
    if (k == prm.nseg - 1 && !prm.sT) {   // nothing after the last segment is needed
      *slot = S;
      break;
    }
    const float4 z = *slot;
    *slot = S;
    const float a = prm.seg_decay[it * prm.dk + row];
    S.x = a * S.x + z.x;
    S.y = a * S.y + z.y;
    S.z = a * S.z + z.z;
    S.w = a * S.w + z.w;
  }
  if (prm.sT) *reinterpret_cast<float4*>(prm.sT + unit * dkdv + e) = S;
}

int launch_seg_scan(const SegScanParams& prm, int units, hipStream_t stream) {
  const int per = prm.dk * prm.dv / 1024;
  hipLaunchKernelGGL(seg_scan_kernel, dim3(units * per), dim3(256), 0, stream, prm);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gla
