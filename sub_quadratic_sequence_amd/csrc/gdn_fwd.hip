// Chunkwise Gated DeltaNet (GDN) forward for gfx950 (MI355X), bf16 inputs,
// fp32 state.
//
// The recurrence (page "Qwen Team Releases FlashQLA for High-Performance
// Linear Attention": GDN's forget gate alpha and update gate beta, one value of
// each per token, and the transition I - beta k k^T):
//     S_t = alpha_t (I - beta_t k_t^T k_t) S_{t-1} + beta_t k_t^T v_t,
//     o_t = q_t S_t.
// Chunkwise (the page's WY steps, with the rewrite that subtracts the state's
// prediction from V before the triangular solve, so no W matrix is formed).
// For a chunk of C = 64 tokens entering with state S, G the in-chunk inclusive
// cumulative log-gate, gamma = exp(G) and Gamma_ij = exp(G_i - G_j):
//     M = I + diag(beta) strict_lower(Gamma * K K^T)      (unit lower triangular)
//     U = M^{-1} diag(beta) (V - diag(gamma) K S)
//     O = diag(gamma) Q S + (Gamma * Q K^T, j <= i) U
//     S <- gamma_C S + (K * exp(G_C - G))^T U
// Every exponential is of a non-positive argument, so no factor exceeds 1.
//
// Work decomposition: one workgroup of 8 waves per (sequence, head, 64-column
// slice of d_v), one producer and one consumer wave per SIMD, over two LDS
// buffers.  The state-independent half of a chunk runs one chunk ahead of the
// state-dependent half:
//  * producer waves 0-3 stage chunk u+1 (q, k rows; the state keys
//    (K exp(G_C - G))^T; V^T; the gates), then compute its score blocks: M
//    (its four 16x16 diagonal blocks in fp32, the rest in bf16) and the causal
//    Gamma * Q K^T;
//  * consumer wave 4 + c owns state columns [16c, 16c+16) for all d_k rows in
//    MFMA accumulators and, for chunk u: the inverse T_cc of M's diagonal block
//    c (fp32 MFMA products of the nilpotent factorisation, shared with the other
//    consumers through LDS), K S and
//    O = gamma Q S, R = beta (V - gamma K S), then the 16-token block forward
//    substitution U_p = T_pp (R_p - sum_{r<p} M_pr U_r) (M^{-1} is never
//    formed), O += P U, and the state update.
// Two workgroup barriers per chunk: the middle one orders the producers'
// staged rows before their score blocks (which read each other's rows) and the
// consumers' inverses before their block solves; the other swaps the buffers.
// The next chunk's raw inputs are loaded into producer registers one chunk ahead.
#include <type_traits>

#include "gla_device.h"
#include "gla_kernels.h"

namespace gla {

namespace gdn {

constexpr int C = 64;
constexpr int DVT = 64;                    // columns per workgroup
constexpr int kBufferFlags = 0x00020000;   // gfx9 buffer descriptor word 3: raw 32-bit dwords
constexpr float kGateFloor = -64.f;        // log-gates below this count as this (alpha = 0 included)

// LDS tiles are dense; their 16- or 8-byte units are permuted within a row by
// XOR with a function of the row, so that the producers' row writes and the
// MFMA fragment reads of a 16-lane group reach distinct banks.
//  * [token][channel] rows (q, k): 16-byte unit u of row r at u ^ f(r)
template <int DK>
__device__ __forceinline__ int tok_off(int r, int ch) {
  const int f = DK == 128 ? (r & 15) : ((r >> 1) & 7);
  return r * DK + (((ch >> 3) ^ f) << 3) + (ch & 7);
}
//  * state keys [channel][token] (128-byte rows, 8-byte units)
__device__ __forceinline__ int kt_off(int r, int tok) {
  const int f = ((r >> 3) & 15) ^ (((r >> 1) & 1) << 2);
  return r * C + (((tok >> 2) ^ f) << 2) + (tok & 3);
}
//  * V^T [column][token]
__device__ __forceinline__ int vt_off(int r, int tok) {
  const int f = ((r >> 2) & 15) ^ (((r >> 1) & 1) << 3);
  return r * C + (((tok >> 2) ^ f) << 2) + (tok & 3);
}
//  * [token][token] tiles (scores, -M)
__device__ __forceinline__ int tt_off(int r, int tok) {
  const int f = (r >> 1) & 7;
  return r * C + (((tok >> 2) ^ f) << 2) + (tok & 3);
}

template <int DK>
struct alignas(16) Buf {
  unsigned short k[C * DK];        // K rows
  unsigned short q[C * DK];        // Q rows
  unsigned short kt[DK * C];       // (K * exp(G_C - G))^T
  unsigned short vt[DVT * C];      // V^T of the slice
  unsigned short p[C * C];         // Gamma * Q K^T for j <= i, zero above the diagonal blocks
  unsigned short mneg[C * C];      // -M below the diagonal blocks
  unsigned short tinv[4][16][20];  // inverses of the diagonal blocks, bf16 [row][col]
  float mdt[4][16][16];            // M's diagonal blocks, strictly lower, fp32, [col][row]
  float gam[C];                    // gamma
  float bet[C];                    // beta
  float g2[C];                     // G in log2 units
};

template <int DK>
struct Smem {
  Buf<DK> b[2];
};

// state-row map (as in the GLA consumer): accumulator tile rb, row r -> key
// channel, chosen so that tiles 2ks and 2ks+1 of a lane hold the 8 consecutive
// channels 32ks + 8gq .. +7 of its column: the state is an MFMA operand as is.
__device__ __forceinline__ int srow(int rb, int r) {
  return 32 * (rb >> 1) + 8 * (r >> 2) + 4 * (rb & 1) + (r & 3);
}

// Workgroup barrier ordering LDS only (outstanding global loads stay in flight).
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 4 + 4 zero slots: a 16-deep contraction on the 32-deep MFMA
__device__ __forceinline__ Frag<BF16> half_frag(uint2 lo) {
  Frag<BF16> f;
  f.v = __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, 0u, 0u});
  return f;
}
__device__ __forceinline__ Frag<BF16> half_frag(const f32x4& x) {
  return half_frag(uint2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])});
}
__device__ __forceinline__ Frag<BF16> pair_frag(const f32x4& a, const f32x4& b) {
  Frag<BF16> f;
  f.v = __builtin_bit_cast(bf16x8, uint4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                         pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])});
  return f;
}
__device__ __forceinline__ Frag<BF16> lds_frag16(const unsigned short* p) {
  Frag<BF16> f;
  f.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
  return f;
}
__device__ __forceinline__ Frag<BF16> lds_frag8x2(const unsigned short* p0, const unsigned short* p1) {
  const uint2 a = *reinterpret_cast<const uint2*>(p0);
  const uint2 b = *reinterpret_cast<const uint2*>(p1);
  Frag<BF16> f;
  f.v = __builtin_bit_cast(bf16x8, uint4{a.x, a.y, b.x, b.y});
  return f;
}
__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace gdn

template <int DK>
__global__ __launch_bounds__(512, 1) void gdn_chunk_fwd_kernel(GdnParams prm) {
  using namespace gdn;
  using BufT = Buf<DK>;
  constexpr int KS = DK / 32;    // 32-channel contraction steps
  constexpr int NRB = DK / 16;   // 16-row state tiles
  constexpr int CPT = DK / 16;   // staging: channels per thread (16 threads per token row)
  constexpr int NW = CPT / 2;    // staging: 32-bit words per token row per thread

  __shared__ Smem<DK> sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, m = lane & 15, gq = lane >> 4;
  const bool producer = wave < 4;

  // ---- work item -----------------------------------------------------------------
  const int bid = blockIdx.x;
  const int lin = prm.xcd_remap ? (bid & 7) * (gridDim.x >> 3) + (bid >> 3) : bid;
  const int unit = lin / prm.nvt;
  const int vt = lin - unit * prm.nvt;
  const int n = unit / prm.H, h = unit - (unit / prm.H) * prm.H;
  long bos, eos, rowbase;
  if (prm.cu) {
    bos = prm.cu[n];
    eos = prm.cu[n + 1];
    rowbase = (long)h * prm.T;
  } else {
    bos = 0;
    eos = prm.T;
    rowbase = ((long)n * prm.H + h) * prm.T;
  }
  const int DV = prm.DV;
  const int vcol0 = vt * DVT;
  const int nch = (int)((eos - bos + C - 1) / C);

  // score blocks above the diagonal blocks are read as zeros by the output product
  for (int i = tid; i < C * C; i += 512) {
    sm.b[0].p[i] = 0;
    sm.b[1].p[i] = 0;
  }

  if (producer) {
    // =========================== producer waves ===========================
    // raw loads: buffer records end at the sequence's last row, so reads past it
    // return zeros (q = k = v = 0, g = beta = 0 on the padding of a last chunk)
    const long r0 = rowbase + bos;
    const int nrow = (int)(eos - bos);
    const int qk_rec = (int)(unsigned)((eos - bos) * DK * 2);   // < 2^32 (host-checked sizes)
    const int v_rec = (int)(unsigned)((eos - bos) * DV * 2);
    const __amdgpu_buffer_rsrc_t rs_q = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(static_cast<const void*>(static_cast<const unsigned short*>(prm.q) + r0 * DK)),
        (short)0, qk_rec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rs_k = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(static_cast<const void*>(static_cast<const unsigned short*>(prm.k) + r0 * DK)),
        (short)0, qk_rec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rs_v = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(static_cast<const void*>(static_cast<const unsigned short*>(prm.v) + r0 * DV)),
        (short)0, v_rec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rs_g = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(static_cast<const void*>(prm.g + r0)), (short)0, nrow * 4, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(static_cast<const void*>(prm.beta + r0)), (short)0, nrow * 4, kBufferFlags);

    // staging roles: thread tid holds tokens 4tg..4tg+3 x channels CPT*cg.. (q, k)
    // and tokens 4tg..4tg+3 x columns 4cg..4cg+3 (v); lane = token for the gates
    const int tg = tid >> 4, cg = tid & 15;
    const unsigned qk_off = (unsigned)((4 * tg) * DK + cg * CPT) * 2u;
    const unsigned v_off = (unsigned)((4 * tg) * DV + vcol0 + 4 * cg) * 2u;
    unsigned rq[4][NW], rk[4][NW], rv[4][2];
    float rg, rb;
    auto load = [&](int u) __attribute__((always_inline)) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const unsigned o = qk_off + (unsigned)(u * C + a) * DK * 2u;
        if constexpr (NW == 4) {
          const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs_q, (int)o, 0, 0);
          const auto y = __builtin_amdgcn_raw_buffer_load_b128(rs_k, (int)o, 0, 0);
#pragma unroll
          for (int j = 0; j < 4; ++j) { rq[a][j] = x[j]; rk[a][j] = y[j]; }
        } else {
          const auto x = __builtin_amdgcn_raw_buffer_load_b64(rs_q, (int)o, 0, 0);
          const auto y = __builtin_amdgcn_raw_buffer_load_b64(rs_k, (int)o, 0, 0);
#pragma unroll
          for (int j = 0; j < 2; ++j) { rq[a][j] = x[j]; rk[a][j] = y[j]; }
        }
        const auto z = __builtin_amdgcn_raw_buffer_load_b64(rs_v, (int)(v_off + (unsigned)(u * C + a) * DV * 2u), 0, 0);
        rv[a][0] = z[0];
        rv[a][1] = z[1];
      }
      rg = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_g, (int)((u * C + lane) * 4), 0, 0));
      rb = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_b, (int)((u * C + lane) * 4), 0, 0));
    };

    // score block D = K_r X_p^T: lane (gq, m) holds k_j . x_t, j = 16r + 4gq + s, t = 16p + m
    auto score = [&](const BufT& B, const unsigned short* xs, int p, int r) __attribute__((always_inline)) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch = 32 * ks + 8 * gq;
        mma(acc, lds_frag16(&B.k[tok_off<DK>(16 * r + m, ch)]), lds_frag16(&xs[tok_off<DK>(16 * p + m, ch)]));
      }
      return acc;
    };

    auto produce = [&](BufT& B, int un) __attribute__((always_inline)) {
      // ---- stage the chunk held in registers ----
      {
        // gates: lane = token; each producer wave scans the chunk for itself
        // (a 16-lane DPP scan, then the totals of the lower rows of 16 added)
        const float b_t = rb;
        float x = fmaxf(rg, kGateFloor) * kLog2e;
        x += dpp<kRowShr1>(x);
        x += dpp<kRowShr2>(x);
        x += dpp<kRowShr4>(x);
        x += dpp<kRowShr8>(x);
        const float r0t = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
        const float r1t = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
        const float r2t = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47));
        const int row16 = lane >> 4;
        x += row16 == 0 ? 0.f : row16 == 1 ? r0t : row16 == 2 ? r0t + r1t : (r0t + r1t) + r2t;
        const float G = x;                       // inclusive, log2 units
        const float Glast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G), 63));
        const float e = fast_exp2(Glast - G);    // key factor of the state update
        if (wave == 0) {
          B.g2[lane] = G;
          B.gam[lane] = fast_exp2(G);
          B.bet[lane] = b_t;
        }
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int row = 4 * tg + a;
          unsigned short* pq = &B.q[tok_off<DK>(row, cg * CPT)];
          unsigned short* pk = &B.k[tok_off<DK>(row, cg * CPT)];
          if constexpr (NW == 4) {
            *reinterpret_cast<uint4*>(pq) = uint4{rq[a][0], rq[a][1], rq[a][2], rq[a][3]};
            *reinterpret_cast<uint4*>(pk) = uint4{rk[a][0], rk[a][1], rk[a][2], rk[a][3]};
          } else {
            *reinterpret_cast<uint2*>(pq) = uint2{rq[a][0], rq[a][1]};
            *reinterpret_cast<uint2*>(pk) = uint2{rk[a][0], rk[a][1]};
          }
        }
        float ef[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) ef[a] = __shfl(e, (4 * tg + a) & 63);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
          float kv[4];
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const unsigned w = rk[a][i >> 1];
            kv[a] = ((i & 1) ? bf_hi(w) : bf_lo(w)) * ef[a];
          }
          store4<BF16>(&B.kt[kt_off(cg * CPT + i, 4 * tg)], kv[0], kv[1], kv[2], kv[3]);
        }
        // V^T: column 4cg + c, tokens 4tg..4tg+3
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int wi = c >> 1;
          const unsigned sel = (c & 1) ? 0x07060302u : 0x05040100u;
          const unsigned lo = __builtin_amdgcn_perm(rv[1][wi], rv[0][wi], sel);
          const unsigned hi = __builtin_amdgcn_perm(rv[3][wi], rv[2][wi], sel);
          *reinterpret_cast<uint2*>(&B.vt[vt_off(4 * cg + c, 4 * tg)]) = uint2{lo, hi};
        }
      }
      load(un);
      barrier_lds();   // (A) every producer's rows are in place

      // ---- scores: wave w takes the M^T blocks (r, p = w), r <= w, and the
      // P^T blocks (r, p = 3 - w), r <= 3 - w: five blocks per wave, block b
      // being M(w, b) for b <= w (b = w: the diagonal block) and P(3 - w, b - w - 1)
      // after; all five products are issued before any is scaled ----
      const int w = wave;
      f32x4 acc[5];
#pragma unroll
      for (int b = 0; b < 5; ++b) {
        const bool is_m = b <= w;
        acc[b] = score(B, is_m ? B.k : B.q, is_m ? w : 3 - w, is_m ? b : b - w - 1);
      }
#pragma unroll
      for (int b = 0; b < 5; ++b) {
        if (b == w) {
          // diagonal block w of M, fp32 [col][row]; the raw block is symmetric, so
          // lane (gq, m) reads it as rows 16w + 4gq + s, column 16w + m
          float mt[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int row = 4 * gq + s;
            mt[s] = (m < row) ? B.bet[16 * w + row] * fast_exp2(B.g2[16 * w + row] - B.g2[16 * w + m]) * acc[b][s]
                              : 0.f;
          }
          *reinterpret_cast<float4*>(&B.mdt[w][m][4 * gq]) = make_float4(mt[0], mt[1], mt[2], mt[3]);
        } else if (b < w) {
          // -M below the diagonal blocks: row t = 16w + m, columns j = 16b + 4gq + s
          const int t = 16 * w + m, j0 = 16 * b + 4 * gq;
          const float gt = B.g2[t], bt = B.bet[t];
          const float4 gj = *reinterpret_cast<const float4*>(&B.g2[j0]);
          store4<BF16>(&B.mneg[tt_off(t, j0)], -bt * fast_exp2(gt - gj.x) * acc[b][0],
                       -bt * fast_exp2(gt - gj.y) * acc[b][1], -bt * fast_exp2(gt - gj.z) * acc[b][2],
                       -bt * fast_exp2(gt - gj.w) * acc[b][3]);
        } else {
          // P = Gamma * Q K^T, j <= t: row t = 16p + m, columns j = 16r + 4gq + s
          const int p = 3 - w, r = b - w - 1;
          const int t = 16 * p + m, j0 = 16 * r + 4 * gq;
          const float gt = B.g2[t];
          const float4 gj = *reinterpret_cast<const float4*>(&B.g2[j0]);
          const float gjs[4] = {gj.x, gj.y, gj.z, gj.w};
          float pv[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) pv[s] = (j0 + s <= t) ? fast_exp2(gt - gjs[s]) * acc[b][s] : 0.f;
          store4<BF16>(&B.p[tt_off(t, j0)], pv[0], pv[1], pv[2], pv[3]);
        }
      }
    };

    if (nch > 0) load(0);
    for (int i = 0; i <= nch; ++i) {
      if (i < nch) {
        produce(sm.b[i & 1], i + 1 < nch ? i + 1 : i);   // clamped look-ahead: no load behind a branch
      } else {
        barrier_lds();   // (A)
      }
      barrier_lds();     // (B) buffer swap
    }
  } else {
    // =========================== consumer waves ===========================
    const int cw = wave - 4;   // state / output columns [16cw, 16cw+16) of the slice
    const float* s_in = prm.s0 ? prm.s0 + (long)unit * DK * DV : nullptr;
    float* s_out = prm.sT ? prm.sT + (long)unit * DK * DV : nullptr;
    f32x4 sacc[NRB];
#pragma unroll
    for (int t = 0; t < NRB; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        sacc[t][s] = s_in ? s_in[(long)srow(t, gq * 4 + s) * DV + vcol0 + cw * 16 + m] : 0.f;
    unsigned short* og = reinterpret_cast<unsigned short*>(prm.o) + rowbase * DV + vcol0 + cw * 16;

    auto consume = [&](BufT& B, int u) __attribute__((always_inline)) {
      // ---- inverse of diagonal block cw of M, fp32: M's diagonal block is I + L
      // with L strictly lower (16 x 16), hence nilpotent, so
      // (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8), eight 16 x 16 x 16
      // products on the 16x16x4 fp32 MFMA.  For a product X Y the operands are
      // X^T and Y as they sit in accumulator layout (lane (gq, m), value s: row
      // 4gq + s, column m): product step s and lane group gq contract index
      // 4gq + s.  L[j][c] = mdt[cw][c][j]. ----
      {
        auto prod = [&](const f32x4& xt, const f32x4& y) __attribute__((always_inline)) {
          f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) d = __builtin_amdgcn_mfma_f32_16x16x4f32(xt[s], y[s], d, 0, 0, 0);
          return d;
        };
        const float4 l4 = *reinterpret_cast<const float4*>(&B.mdt[cw][m][4 * gq]);
        const f32x4 Lc = f32x4{l4.x, l4.y, l4.z, l4.w};   // L
        f32x4 LTc, Ic;                                      // L^T, I
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          LTc[s] = B.mdt[cw][4 * gq + s][m];
          Ic[s] = (4 * gq + s == m) ? 1.f : 0.f;
        }
        const f32x4 L2 = prod(LTc, Lc), L2T = prod(Lc, LTc);
        const f32x4 L4 = prod(L2T, L2), L4T = prod(L2, L2T);
        const f32x4 L8 = prod(L4T, L4);
        // T^T = (I + L^8)^T (I + L^4)^T (I + L^2)^T (I - L)^T, from the right
        f32x4 z = Ic - LTc;
        z = prod(Ic + L2, z);
        z = prod(Ic + L4, z);
        z = prod(Ic + L8, z);
        // z is T^T in accumulator layout: lane (gq, m) holds T[m][4gq .. 4gq + 3]
        *reinterpret_cast<uint2*>(&B.tinv[cw][m][4 * gq]) =
            uint2{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])};
      }
      // ---- K S (tokens x columns), then R ----
      f32x4 r_acc[4], o_acc[4];
      Frag<BF16> sf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sf[ks] = pair_frag(sacc[2 * ks], sacc[2 * ks + 1]);
      {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          r_acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            mma(r_acc[p], lds_frag16(&B.k[tok_off<DK>(16 * p + m, 32 * ks + 8 * gq)]), sf[ks]);
          // R = beta (V - gamma K S): rows t = 16p + 4gq + s, column 16cw + m
          const float4 bt = *reinterpret_cast<const float4*>(&B.bet[16 * p + 4 * gq]);
          const float4 gm = *reinterpret_cast<const float4*>(&B.gam[16 * p + 4 * gq]);
          const uint2 vw = *reinterpret_cast<const uint2*>(&B.vt[vt_off(16 * cw + m, 16 * p + 4 * gq)]);
          r_acc[p][0] = bt.x * (bf_lo(vw.x) - gm.x * r_acc[p][0]);
          r_acc[p][1] = bt.y * (bf_hi(vw.x) - gm.y * r_acc[p][1]);
          r_acc[p][2] = bt.z * (bf_lo(vw.y) - gm.z * r_acc[p][2]);
          r_acc[p][3] = bt.w * (bf_hi(vw.y) - gm.w * r_acc[p][3]);
        }
      }
      barrier_lds();   // (A) every consumer's inverse is in place
      // ---- O^T = gamma S^T Q^T (issued beside the block solve's dependent chain) ----
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        o_acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          mma(o_acc[p], sf[ks], lds_frag16(&B.q[tok_off<DK>(16 * p + m, 32 * ks + 8 * gq)]));
      }
      // ---- U_p = T_pp (R_p - sum_{r<p} M_pr U_r): 16-deep products ----
      f32x4 uacc[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        f32x4 x = r_acc[p];
#pragma unroll
        for (int r = 0; r < p; ++r)
          mma(x, half_frag(*reinterpret_cast<const uint2*>(&B.mneg[tt_off(16 * p + m, 16 * r + 4 * gq)])),
              half_frag(uacc[r]));
        uacc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
        mma(uacc[p], half_frag(*reinterpret_cast<const uint2*>(&B.tinv[p][m][4 * gq])), half_frag(x));
      }
      // U as an operand: slots = tokens 32j + 4gq + s and 32j + 16 + 4gq + s
      Frag<BF16> uf[2];
      uf[0] = pair_frag(uacc[0], uacc[1]);
      uf[1] = pair_frag(uacc[2], uacc[3]);
      // ---- O^T(column 4gq + s, query 16p + m) = gamma_t S^T Q^T + U^T P^T, store ----
      const long t0 = bos + (long)u * C;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float gt = B.gam[16 * p + m];
#pragma unroll
        for (int s = 0; s < 4; ++s) o_acc[p][s] *= gt;
#pragma unroll
        for (int j = 0; 2 * j <= p; ++j) {
          const int row = 16 * p + m;
          mma(o_acc[p], uf[j], lds_frag8x2(&B.p[tt_off(row, 32 * j + 4 * gq)], &B.p[tt_off(row, 32 * j + 16 + 4 * gq)]));
        }
        const long t = t0 + 16 * p + m;
        if (t < eos) store4<BF16>(og + t * DV + 4 * gq, o_acc[p][0], o_acc[p][1], o_acc[p][2], o_acc[p][3]);
      }
      // ---- S <- gamma_C S + Khat^T U ----
      const float gC = B.gam[C - 1];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
        for (int s = 0; s < 4; ++s) sacc[rb][s] *= gC;
        const int row = srow(rb, m);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          mma(sacc[rb], lds_frag8x2(&B.kt[kt_off(row, 32 * j + 4 * gq)], &B.kt[kt_off(row, 32 * j + 16 + 4 * gq)]),
              uf[j]);
      }
    };

    for (int i = 0; i <= nch; ++i) {
      if (i > 0) {
        consume(sm.b[(i - 1) & 1], i - 1);
      } else {
        barrier_lds();   // (A)
      }
      barrier_lds();     // (B) buffer swap
    }
    if (s_out) {
#pragma unroll
      for (int t = 0; t < NRB; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          s_out[(long)srow(t, gq * 4 + s) * DV + vcol0 + cw * 16 + m] = sacc[t][s];
    }
  }
}

int launch_gdn_chunk_fwd(const GdnParams& prm, int dk, int nblocks, hipStream_t stream) {
  if (dk == 128) {
    hipLaunchKernelGGL((gdn_chunk_fwd_kernel<128>), dim3(nblocks), dim3(512), 0, stream, prm);
  } else if (dk == 64) {
    hipLaunchKernelGGL((gdn_chunk_fwd_kernel<64>), dim3(nblocks), dim3(512), 0, stream, prm);
  } else {
    return -2;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gla
