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
// Work decomposition: one workgroup of 4 waves per (sequence, head, 64-column
// slice of d_v).  Wave w owns state columns [16w, 16w+16) of the slice for all
// d_k rows in MFMA accumulators; it computes its columns of K S, U, O and the
// state update.  The chunk-wide pieces (score blocks, the inverses of the four
// 16x16 diagonal blocks of M) are split across the waves through LDS.
// M^{-1} is never formed whole: each wave solves M U = R by 16-token block
// forward substitution, U_p = T_pp (R_p - sum_{r<p} M_pr U_r), with T_pp the
// inverse of diagonal block p.
//
// Per chunk: stage the tiles | scores, K S, S^T Q^T, R | diagonal inverses |
// block solve, outputs, state update - four workgroup barriers.  The next
// chunk's raw q, k, v, g, beta are loaded into registers one chunk ahead.
#include "gla_device.h"
#include "gla_kernels.h"

namespace gla {

namespace gdn {

constexpr int C = 64;
constexpr int DVT = 64;                    // columns per workgroup
constexpr int kBufferFlags = 0x00020000;   // gfx9 buffer descriptor word 3: raw 32-bit dwords
constexpr float kGateFloor = -64.f;        // log-gates below this count as this (alpha = 0 included)

template <int DK>
struct alignas(16) Smem {
  static constexpr int PK = DK + 8;        // [token][channel] pitch (elements)
  static constexpr int PT = C + 8;         // [channel | column | token][token] pitch
  unsigned short k[C * PK];                // K rows
  unsigned short q[C * PK];                // Q rows
  unsigned short kt[DK * PT];              // (K * exp(G_C - G))^T  [channel][token]
  unsigned short vt[DVT * PT];             // V^T of the slice      [column][token]
  unsigned short p[C * PT];                // Gamma * Q K^T, j <= i  [query][key]
  unsigned short mneg[C * PT];             // -M below the diagonal blocks [row][col]
  unsigned short tinv[4][16][24];          // inverses of the diagonal blocks, bf16 [row][col]
  float mdt[4][16][20];                    // strictly-lower diagonal blocks of M, fp32, [col][row]
  float g2[C];                             // G in log2 units
  float gam[C];                            // gamma
  float bet[C];                            // beta
};

// state-row map (as in the GLA consumer): accumulator tile rb, row r -> key
// channel, chosen so that tiles 2ks and 2ks+1 of a lane hold the 8 consecutive
// channels 32ks + 8gq .. +7 of its column: the state is an MFMA operand as is.
__device__ __forceinline__ int srow(int rb, int r) {
  return 32 * (rb >> 1) + 8 * (r >> 2) + 4 * (rb & 1) + (r & 3);
}

__device__ __forceinline__ void barrier() { __syncthreads(); }

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

}  // namespace gdn

template <int DK>
__global__ __launch_bounds__(256, 1) void gdn_chunk_fwd_kernel(GdnParams prm) {
  using namespace gdn;
  using SM = Smem<DK>;
  constexpr int PK = SM::PK, PT = SM::PT;
  constexpr int KS = DK / 32;    // 32-channel contraction steps
  constexpr int NRB = DK / 16;   // 16-row state tiles
  constexpr int CPT = DK / 16;   // staging: channels per thread (16 threads per token row)
  constexpr int NW = CPT / 2;    // staging: 32-bit words per token row per thread

  __shared__ SM sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, m = lane & 15, gq = lane >> 4;

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
  const float* s_in = prm.s0 ? prm.s0 + (long)unit * DK * DV : nullptr;
  float* s_out = prm.sT ? prm.sT + (long)unit * DK * DV : nullptr;

  // ---- raw loads: buffer records end at the sequence's last row, so reads past
  // it return zeros (q = k = v = 0, g = beta = 0 on the padding of a last chunk)
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
  // and tokens 4tg..4tg+3 x columns 4cg..4cg+3 (v)
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

  // ---- state: wave w owns columns [16w, 16w+16) of the slice, all DK rows
  f32x4 sacc[NRB];
#pragma unroll
  for (int t = 0; t < NRB; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      sacc[t][s] = s_in ? s_in[(long)srow(t, gq * 4 + s) * DV + vcol0 + wave * 16 + m] : 0.f;

  // score blocks above the diagonal blocks are read as zeros by the output product
  for (int i = tid; i < C * PT; i += 256) sm.p[i] = 0;

  unsigned short* og = reinterpret_cast<unsigned short*>(prm.o) + rowbase * DV + vcol0 + wave * 16;
  if (nch > 0) load(0);

  for (int u = 0; u < nch; ++u) {
    // ============ 1. stage the chunk ============
    {
      // gates: lane = token; every wave scans the chunk (no cross-wave step needed)
      const float b_t = rb;
      float x = fmaxf(rg, kGateFloor) * kLog2e;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_up(x, d);
        x += lane >= d ? y : 0.f;
      }
      const float G = x;                       // inclusive, log2 units
      const float Glast = __shfl(G, 63);
      const float e = fast_exp2(Glast - G);    // key factor of the state update
      if (wave == 0) {
        sm.g2[lane] = G;
        sm.gam[lane] = fast_exp2(G);
        sm.bet[lane] = b_t;
      }
      // q, k rows as they are; k scaled by exp(G_C - G_t) transposed into kt
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        unsigned short* pq = &sm.q[(4 * tg + a) * PK + cg * CPT];
        unsigned short* pk = &sm.k[(4 * tg + a) * PK + cg * CPT];
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
          kv[a] = ((i & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16)) * ef[a];
        }
        store4<BF16>(&sm.kt[(cg * CPT + i) * PT + 4 * tg], kv[0], kv[1], kv[2], kv[3]);
      }
      // V^T: column 4cg + c, tokens 4tg..4tg+3
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int wi = c >> 1;
        const unsigned sel = (c & 1) ? 0x07060302u : 0x05040100u;
        const unsigned lo = __builtin_amdgcn_perm(rv[1][wi], rv[0][wi], sel);
        const unsigned hi = __builtin_amdgcn_perm(rv[3][wi], rv[2][wi], sel);
        *reinterpret_cast<uint2*>(&sm.vt[(4 * cg + c) * PT + 4 * tg]) = uint2{lo, hi};
      }
    }
    if (u + 1 < nch) load(u + 1);
    barrier();

    // ============ 2. scores, K S, S^T Q^T, R ============
    // wave w: the M^T blocks (r, p = w), r <= w, and the P^T blocks (r, p = 3 - w),
    // r <= 3 - w: five blocks per wave
    {
      auto score_block = [&](bool is_m, int p, int r) __attribute__((always_inline)) {
        // D = K_r X_p^T: lane (gq, m) holds k_j . x_t, j = 16r + 4gq + s, t = 16p + m
        const unsigned short* xs = is_m ? sm.k : sm.q;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const Frag<BF16> a = lds_frag16(&sm.k[(16 * r + m) * PK + 32 * ks + 8 * gq]);
          const Frag<BF16> b = lds_frag16(&xs[(16 * p + m) * PK + 32 * ks + 8 * gq]);
          mma(acc, a, b);
        }
        const int t = 16 * p + m;
        const int j0 = 16 * r + 4 * gq;
        const float gt = sm.g2[t];
        const float4 gj = *reinterpret_cast<const float4*>(&sm.g2[j0]);
        const float gjs[4] = {gj.x, gj.y, gj.z, gj.w};
        if (is_m) {
          const float bt = sm.bet[t];
          float mv[4];
#pragma unroll
          for (int s = 0; s < 4; ++s)
            mv[s] = (j0 + s < t) ? bt * fast_exp2(gt - gjs[s]) * acc[s] : 0.f;
          if (r == p) {
            // diagonal block, fp32, stored [col][row]: mdt[p][t % 16][j % 16]
            // (the raw block is symmetric: read it as rows j, column t)
            float mt[4];
            const int jr = 4 * gq;          // this lane's rows 16p + 4gq + s of M, column m
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const int row = jr + s;
              const float gr = sm.g2[16 * p + row];
              mt[s] = (m < row) ? sm.bet[16 * p + row] * fast_exp2(gr - sm.g2[16 * p + m]) * acc[s] : 0.f;
            }
            *reinterpret_cast<float4*>(&sm.mdt[p][m][jr]) = make_float4(mt[0], mt[1], mt[2], mt[3]);
          } else {
            store4<BF16>(&sm.mneg[t * PT + j0], -mv[0], -mv[1], -mv[2], -mv[3]);
          }
        } else {
          float pv[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) pv[s] = (j0 + s <= t) ? fast_exp2(gt - gjs[s]) * acc[s] : 0.f;
          store4<BF16>(&sm.p[t * PT + j0], pv[0], pv[1], pv[2], pv[3]);
        }
      };
      for (int r = 0; r <= wave; ++r) score_block(true, wave, r);
      for (int r = 0; r <= 3 - wave; ++r) score_block(false, 3 - wave, r);
    }
    // K S (tokens x this wave's columns) and O^T = S^T Q^T, from the state entering the chunk
    f32x4 ks_acc[4], o_acc[4];
    {
      Frag<BF16> sf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sf[ks] = pair_frag(sacc[2 * ks], sacc[2 * ks + 1]);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        ks_acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
        o_acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          mma(ks_acc[p], lds_frag16(&sm.k[(16 * p + m) * PK + 32 * ks + 8 * gq]), sf[ks]);
          mma(o_acc[p], sf[ks], lds_frag16(&sm.q[(16 * p + m) * PK + 32 * ks + 8 * gq]));
        }
        // O^T(column 4gq + s, token 16p + m) *= gamma_t
        const float gt = sm.gam[16 * p + m];
#pragma unroll
        for (int s = 0; s < 4; ++s) o_acc[p][s] *= gt;
        // R = beta (V - gamma K S): rows t = 16p + 4gq + s, column 16w + m
        const float4 bt = *reinterpret_cast<const float4*>(&sm.bet[16 * p + 4 * gq]);
        const float4 gm = *reinterpret_cast<const float4*>(&sm.gam[16 * p + 4 * gq]);
        const uint2 vw = *reinterpret_cast<const uint2*>(&sm.vt[(16 * wave + m) * PT + 16 * p + 4 * gq]);
        const float vv[4] = {__uint_as_float(vw.x << 16), __uint_as_float(vw.x & 0xffff0000u),
                             __uint_as_float(vw.y << 16), __uint_as_float(vw.y & 0xffff0000u)};
        const float bs[4] = {bt.x, bt.y, bt.z, bt.w}, gs[4] = {gm.x, gm.y, gm.z, gm.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) ks_acc[p][s] = bs[s] * (vv[s] - gs[s] * ks_acc[p][s]);
      }
    }
    barrier();

    // ============ 3. inverse of diagonal block p = w (fp32, row per lane) ============
    {
      // T (I + L) = I: row i of T from its last column to its first,
      // T[i][c] = [c == i] - sum_{j > c} T[i][j] L[j][c]; L[j][c] = mdt[w][c][j]
      const int i = m;
      float t[16];
#pragma unroll
      for (int c = 15; c >= 0; --c) {
        float acc = (c == i) ? 1.f : 0.f;
#pragma unroll
        for (int j = c + 1; j < 16; ++j) acc -= t[j] * sm.mdt[wave][c][j];
        t[c] = acc;
      }
      if (gq == 0) {
        uint4 lo = {pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3]), pack_bf16x2(t[4], t[5]),
                    pack_bf16x2(t[6], t[7])};
        uint4 hi = {pack_bf16x2(t[8], t[9]), pack_bf16x2(t[10], t[11]), pack_bf16x2(t[12], t[13]),
                    pack_bf16x2(t[14], t[15])};
        *reinterpret_cast<uint4*>(&sm.tinv[wave][i][0]) = lo;
        *reinterpret_cast<uint4*>(&sm.tinv[wave][i][8]) = hi;
      }
    }
    barrier();

    // ============ 4. block solve, outputs, state ============
    {
      // U_p = T_pp (R_p - sum_{r<p} M_pr U_r), 16-deep products (4 real slots per lane)
      f32x4 uacc[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        f32x4 x = ks_acc[p];
#pragma unroll
        for (int r = 0; r < p; ++r) {
          const Frag<BF16> a = half_frag(*reinterpret_cast<const uint2*>(&sm.mneg[(16 * p + m) * PT + 16 * r + 4 * gq]));
          mma(x, a, half_frag(uacc[r]));
        }
        uacc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
        mma(uacc[p], half_frag(*reinterpret_cast<const uint2*>(&sm.tinv[p][m][4 * gq])), half_frag(x));
      }
      // U as an operand: slots = tokens 32j + 4gq + s and 32j + 16 + 4gq + s
      Frag<BF16> uf[2];
      uf[0] = pair_frag(uacc[0], uacc[1]);
      uf[1] = pair_frag(uacc[2], uacc[3]);
      // O^T += U^T P^T (queries 16p + m)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
#pragma unroll
        for (int j = 0; 2 * j <= p; ++j) {
          const unsigned short* pr = &sm.p[(16 * p + m) * PT + 32 * j + 4 * gq];
          mma(o_acc[p], uf[j], lds_frag8x2(pr, pr + 16));
        }
        const long t = bos + (long)u * C + 16 * p + m;
        if (t < eos) store4<BF16>(og + t * DV + 4 * gq, o_acc[p][0], o_acc[p][1], o_acc[p][2], o_acc[p][3]);
      }
      // S <- gamma_C S + Khat^T U
      const float gC = sm.gam[C - 1];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
        for (int s = 0; s < 4; ++s) sacc[rb][s] *= gC;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const unsigned short* kr = &sm.kt[srow(rb, m) * PT + 32 * j + 4 * gq];
          mma(sacc[rb], lds_frag8x2(kr, kr + 16), uf[j]);
        }
      }
    }
    barrier();
  }

  if (s_out) {
#pragma unroll
    for (int t = 0; t < NRB; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        s_out[(long)srow(t, gq * 4 + s) * DV + vcol0 + wave * 16 + m] = sacc[t][s];
  }
}

int launch_gdn_chunk_fwd(const GdnParams& prm, int dk, int nblocks, hipStream_t stream) {
  if (dk == 128) {
    hipLaunchKernelGGL((gdn_chunk_fwd_kernel<128>), dim3(nblocks), dim3(256), 0, stream, prm);
  } else if (dk == 64) {
    hipLaunchKernelGGL((gdn_chunk_fwd_kernel<64>), dim3(nblocks), dim3(256), 0, stream, prm);
  } else {
    return -2;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gla
