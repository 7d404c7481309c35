// Single-token GLA decode step for gfx950 (MI355X).
//
// One token of the recurrence of the page "Gated Linear Attention (GLA):
// Mathematical Foundations ...", section "The Gated Recurrent Update", per
// (sequence, head): S = diag(exp(g)) S + k^T v, then o = q S with the updated
// S (the constant-memory decode step of the FlashLinearAttention page,
// section "The O(1) Inference Memory Revolution").
//
// The step is bound by HBM: the fp32 d_k x d_v state is read and written once
// (8 d_k d_v bytes) for 5 d_k d_v flops.  One 256-lane workgroup streams one
// unit's state: lane (cg, rg) owns columns 4cg..4cg+3 of the rows
// rg, rg + RG, rg + 2 RG, ... so every 16-byte load and store of a state row
// is coalesced across the row's column groups, and each lane has all its row
// loads in flight before it updates and stores them.  alpha = 2^(g log2 e),
// q and k are staged once per unit in LDS; o is reduced across the row groups
// through LDS in a fixed order.
#include "gla_device.h"
#include "gla_kernels.h"

namespace gla {

template <int DK, int DV, typename E>
__global__ __launch_bounds__(256) void recurrent_step_kernel(StepParams prm) {
  using S = typename E::storage;
  constexpr int CG = DV / 4;          // column groups of 4
  constexpr int RG = 256 / CG;        // row groups
  constexpr int RPT = DK / RG;        // rows per lane
  constexpr int BATCH = RPT < 16 ? RPT : 16;
  static_assert(RPT % BATCH == 0, "rows per lane");

  __shared__ float s_a[DK], s_k[DK], s_q[DK];
  __shared__ float s_red[RG][DV + 4];

  const int unit = blockIdx.x;
  const int tid = threadIdx.x;
  const S* qg = reinterpret_cast<const S*>(prm.q) + (long)unit * DK;
  const S* kg = reinterpret_cast<const S*>(prm.k) + (long)unit * DK;
  const S* gg = reinterpret_cast<const S*>(prm.g) + (long)unit * DK;
  const S* vg = reinterpret_cast<const S*>(prm.v) + (long)unit * DV;
  S* og = reinterpret_cast<S*>(prm.o) + (long)unit * DV;
  float* st = prm.state + (long)unit * DK * DV;

  for (int i = tid; i < DK; i += 256) {
    float gv, kv, qv;
    if constexpr (E::kBytes == 2) {
      gv = bf16_bits_to_f32(gg[i]);
      kv = bf16_bits_to_f32(kg[i]);
      qv = bf16_bits_to_f32(qg[i]);
    } else {
      gv = gg[i];
      kv = kg[i];
      qv = qg[i];
    }
    s_a[i] = fast_exp2(gv * kLog2e);
    s_k[i] = kv;
    s_q[i] = qv;
  }
  const int cg = tid % CG, rg = tid / CG;
  float v[4];
  load_vec<E, 4>(vg + 4 * cg, v);
  __syncthreads();

  float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
  for (int b0 = 0; b0 < RPT; b0 += BATCH) {
    float4 sv[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int r = rg + RG * (b0 + i);
      sv[i] = *reinterpret_cast<const float4*>(st + (long)r * DV + 4 * cg);
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int r = rg + RG * (b0 + i);
      const float a = s_a[r], kr = s_k[r], qr = s_q[r];
      float4 x = sv[i];
      x.x = a * x.x + kr * v[0];
      x.y = a * x.y + kr * v[1];
      x.z = a * x.z + kr * v[2];
      x.w = a * x.w + kr * v[3];
      *reinterpret_cast<float4*>(st + (long)r * DV + 4 * cg) = x;
      o0 += qr * x.x;
      o1 += qr * x.y;
      o2 += qr * x.z;
      o3 += qr * x.w;
    }
  }
  s_red[rg][4 * cg + 0] = o0;
  s_red[rg][4 * cg + 1] = o1;
  s_red[rg][4 * cg + 2] = o2;
  s_red[rg][4 * cg + 3] = o3;
  __syncthreads();
  if (tid < CG) {
    float acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < RG; ++r) s += s_red[r][4 * tid + c];
      acc[c] = s;
    }
    store4<E>(og + 4 * tid, acc[0], acc[1], acc[2], acc[3]);
  }
}

template <int DK, int DV, typename E>
static int launch_step(const StepParams& prm, int units, hipStream_t stream) {
  hipLaunchKernelGGL((recurrent_step_kernel<DK, DV, E>), dim3(units), dim3(256), 0, stream, prm);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <typename E>
static int dispatch_step(const StepParams& prm, int units, int dk, int dv, hipStream_t stream) {
#define GLA_STEP_CASE(DKV, DVV) \
  if (dk == DKV && dv == DVV) return launch_step<DKV, DVV, E>(prm, units, stream);
  GLA_STEP_CASE(64, 64) GLA_STEP_CASE(64, 128) GLA_STEP_CASE(64, 256)
  GLA_STEP_CASE(128, 64) GLA_STEP_CASE(128, 128) GLA_STEP_CASE(128, 256)
  GLA_STEP_CASE(256, 64) GLA_STEP_CASE(256, 128) GLA_STEP_CASE(256, 256)
#undef GLA_STEP_CASE
  return -2;
}

int launch_recurrent_step(const StepParams& prm, int units, int dk, int dv, int dtype,
                          hipStream_t stream) {
  if (dtype == 0) return dispatch_step<BF16>(prm, units, dk, dv, stream);
  if (dtype == 1) return dispatch_step<F32>(prm, units, dk, dv, stream);
  return -2;
}

}  // namespace gla
