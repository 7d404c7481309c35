// Chunkwise-parallel GLA forward for gfx950 (MI355X).
//
// Implements the chunk form of the page "Gated Linear Attention (GLA):
// Mathematical Foundations ...", sections "Sequence Partitioning and State
// Factorization" and "Mathematical Formulation of Chunk Computations": per chunk
// of C = 64 tokens, Gamma = inclusive cumulative sum of log alpha inside the
// chunk; O = ((Q K^T) with the channel-wise decay exp(Gamma_i - Gamma_j), j <= i) V
// + (Q * exp(Gamma)) S_prev; S = diag(exp(Gamma_last)) S_prev
// + (K * exp(Gamma_last - Gamma))^T V.  The decay "D" that the page writes as a
// C x C mask is per key channel for GLA, so it is applied inside the sum over
// channels (through the operand scalings below).
//
// Work decomposition: one workgroup (4 waves, 256 lanes) per (sequence, head,
// 64-column slice of d_v).  The columns of S evolve independently, so the
// slices need no communication; the workgroup walks its sequence's chunks in
// order with the fp32 state slice resident in MFMA accumulators.
//
// Per chunk:
//  1. gating (all lanes): lane (tg = lane%16, gq = lane/16) of wave w holds
//     tokens 4tg..4tg+3 and key channels w*DK/4 + gq*DK/16 .. + DK/16.  The
//     log2-gate cumulative sum is a serial sum over the lane's 4 tokens plus a
//     DPP scan over the 16 lanes of its row, so the whole chunk is scanned
//     without leaving the wave.  Exponentials are exp2 of log2-scaled gates.
//  2. operand tiles are written to LDS in the layouts the MFMAs read:
//     QE = Q * 2^Gamma (inter term), KP (key operand of the scores), KT = the
//     state-update keys K * 2^(Gamma_last - Gamma) stored channel-major, VT = V
//     stored column-major, SBT = the previous state, column-major.
//  3. MFMA (v_mfma_f32_16x16x32_bf16, or 16x16x4 f32): wave p computes the
//     transposed score blocks P^T(r, p), r <= p, of its 16-query sub-chunk p;
//     then O^T = V^T P^T + S_prev^T (Q*2^Gamma)^T for its 16 queries; then the
//     state update of its DK/4 channels: S = diag(2^Gamma_last) S + KT VT^T.
//
// Numerical safety of exp(Gamma_i - Gamma_j): gates are <= 0, so Gamma falls
// inside a chunk.  Two factorisations of exp(Gamma_i - Gamma_j) into a query
// factor and a key factor are used, chosen per chunk:
//  * single pivot (chunk start) when the chunk's total decay is at most 2^60:
//    P = (Q 2^Gamma)(K 2^-Gamma)^T; every factor stays within [2^-60, 2^60].
//  * sub-chunk pivots (16-token sub-chunks) otherwise: with B_p = Gamma at the
//    row before sub-chunk p, Qh = Q 2^(Gamma - B_p) <= |Q| and
//    Kt = K 2^(B_{r+1} - Gamma) <= |K|; block (p, r) uses
//    Qh diag(2^(B_p - B_{r+1})) Kt^T.  Off-diagonal factors are all <= 1 (an
//    underflow only drops a term whose true value is below it); the diagonal
//    block needs 2^(B_p - B_{p+1}) = 2^(decay over 16 tokens), which is exact
//    while that decay is below 2^100.  Beyond it the diagonal block is
//    computed element by element on the VALU, exp2 of each gate difference.
#include "gla_device.h"
#include "gla_kernels.h"

namespace gla {

template <int DK, typename E>
struct ChunkCfg {
  static constexpr int C = 64;             // chunk length
  static constexpr int DVT = 64;           // d_v columns per workgroup
  static constexpr int CPL = DK / 16;      // gating: key channels per lane
  static constexpr int WCH = DK / 4;       // key channels per wave
  static constexpr int KS = DK / 32;       // 32-wide contraction steps over channels
  static constexpr int RB = DK / 64;       // 16-row blocks of S per wave
  static constexpr int PADE = 16 / E::kBytes;
  static constexpr int PQ = DK + PADE;     // pitch of [token][channel] and [col][channel] tiles
  static constexpr int PT = C + PADE;      // pitch of [channel|col][token] tiles
  static constexpr int NW_QKG = CPL * E::kBytes / 4;  // 32-bit words per lane per token
  static constexpr int NW_V = 4 * E::kBytes / 4;
  // LDS tiles (in elements)
  static constexpr int SZ_QE = C * PQ;
  static constexpr int SZ_KP = C * PQ;
  static constexpr int SZ_QP = 10 * 16 * PQ;   // sub-chunk-pivot query copies, one per block (p, r<=p)
  static constexpr int SZ_KT = DK * PT;
  static constexpr int SZ_VT = DVT * PT;
  static constexpr int SZ_SB = DVT * PQ;
};

template <int NW>
struct Raw {
  unsigned w[NW];
};

template <int NW>
__device__ __forceinline__ void raw_load(Raw<NW>& r, const void* p) {
  if constexpr (NW == 4) {
    uint4 x = *reinterpret_cast<const uint4*>(p);
    r.w[0] = x.x; r.w[1] = x.y; r.w[2] = x.z; r.w[3] = x.w;
  } else if constexpr (NW == 2) {
    uint2 x = *reinterpret_cast<const uint2*>(p);
    r.w[0] = x.x; r.w[1] = x.y;
  } else {
    static_assert(NW == 8, "raw width");
    uint4 x = reinterpret_cast<const uint4*>(p)[0];
    uint4 y = reinterpret_cast<const uint4*>(p)[1];
    r.w[0] = x.x; r.w[1] = x.y; r.w[2] = x.z; r.w[3] = x.w;
    r.w[4] = y.x; r.w[5] = y.y; r.w[6] = y.z; r.w[7] = y.w;
  }
}
template <int NW>
__device__ __forceinline__ void raw_zero(Raw<NW>& r) {
#pragma unroll
  for (int i = 0; i < NW; ++i) r.w[i] = 0u;
}

// Unpack N elements held in a Raw into floats.
template <typename E, int N, int NW>
__device__ __forceinline__ void raw_unpack(const Raw<NW>& r, float* out) {
  if constexpr (E::kBytes == 2) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      out[2 * i] = __uint_as_float(r.w[i] << 16);
      out[2 * i + 1] = __uint_as_float(r.w[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = __uint_as_float(r.w[i]);
  }
}

__device__ __forceinline__ float clamp_gate(float x) {
  // log2-gate floor: 2^-256 is already 0 in fp32, so this changes no finite
  // result; it keeps g = -inf (alpha = 0) from producing inf - inf.  NaN passes.
  return x < -256.f ? -256.f : x;
}

template <int DK, typename E>
__global__ __launch_bounds__(256, 1) void chunk_fwd_kernel(ChunkParams prm) {
  // The chunk is processed in NH passes of 64 key channels each (DK = 64: one
  // pass).  Scores and the inter-chunk term are sums over channels, so each
  // pass adds its channels' share to the same accumulators; the state rows of
  // a pass's channels are updated in that pass.  P V and the output store
  // follow the last pass.  The LDS tiles are sized for one pass.
  constexpr int DKH = 64, NH = DK / DKH;
  static_assert(DK % DKH == 0, "d_k is a multiple of 64");
  using Cfg = ChunkCfg<DKH, E>;
  using S = typename E::storage;
  constexpr int C = Cfg::C, CPL = Cfg::CPL, WCH = Cfg::WCH, KS = Cfg::KS;
  constexpr int PQ = Cfg::PQ, PT = Cfg::PT;
  static_assert(Cfg::RB == 1, "one 16-row state block per wave and pass");

  __shared__ __attribute__((aligned(16))) S s_qe[Cfg::SZ_QE];
  __shared__ __attribute__((aligned(16))) S s_kp[Cfg::SZ_KP];
  __shared__ __attribute__((aligned(16))) S s_qp[Cfg::SZ_QP];
  __shared__ __attribute__((aligned(16))) S s_kt[Cfg::SZ_KT];
  __shared__ __attribute__((aligned(16))) S s_vt[Cfg::SZ_VT];
  __shared__ __attribute__((aligned(16))) S s_sb[Cfg::SZ_SB];
  __shared__ float s_dec[DKH];                // 2^Gamma_last per key channel of the pass
  __shared__ float s_diag[4][4][16][16];      // [sub-chunk][wave][i][j] exact diagonal partials
  __shared__ int s_flag[2][4];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, m = lane & 15, gq = lane >> 4;

  // ---- work item: (sequence n, head h, d_v slice vt) ----------------------------
  const int nblk = gridDim.x;
  const int bid = blockIdx.x;
  const int lin = prm.xcd_remap ? (bid & 7) * (nblk >> 3) + (bid >> 3) : bid;
  const int unit = lin / prm.nvt, vt = lin - unit * prm.nvt;
  const int n = unit / prm.H, hd = unit - n * prm.H;
  long bos, eos, rowbase;
  if (prm.cu) {
    bos = prm.cu[n];
    eos = prm.cu[n + 1];
    rowbase = (long)hd * prm.T;
  } else {
    bos = 0;
    eos = prm.T;
    rowbase = ((long)n * prm.H + hd) * prm.T;
  }
  const int DV = prm.DV;
  const S* qg = reinterpret_cast<const S*>(prm.q) + rowbase * DK;
  const S* kg = reinterpret_cast<const S*>(prm.k) + rowbase * DK;
  const S* gg = reinterpret_cast<const S*>(prm.g) + rowbase * DK;
  const S* vg = reinterpret_cast<const S*>(prm.v) + rowbase * DV;
  S* og = reinterpret_cast<S*>(prm.o) + rowbase * DV;
  const int vcol0 = vt * Cfg::DVT;
  const long sbase = (long)unit * DK * DV;

  // ---- state slice: in pass ph, wave w owns key channels 64 ph + [w*WCH, (w+1)*WCH) x 64 columns
  f32x4 sacc[NH][4];
#pragma unroll
  for (int ph = 0; ph < NH; ++ph)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c = DKH * ph + w * WCH + gq * 4 + s;
        sacc[ph][cb][s] = prm.s0 ? prm.s0[sbase + (long)c * DV + vcol0 + cb * 16 + m] : 0.f;
      }

  // ---- gating lane geometry -----------------------------------------------------
  const int tg = m;                       // token group: tokens 4tg..4tg+3 of the chunk
  const int ch0 = w * WCH + gq * CPL;     // first key channel of this lane within a pass
  const int sub = tg >> 2;                // 16-token sub-chunk of these tokens
  const int vc0 = w * 16 + gq * 4;        // first of this lane's 4 V columns (of the slice)

  Raw<Cfg::NW_QKG> rq[NH][4], rk[NH][4], rg[NH][4];
  Raw<Cfg::NW_V> rv[4];

  auto prefetch = [&](long t0) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const long t = t0 + 4 * tg + a;
      if (t < eos) {
#pragma unroll
        for (int ph = 0; ph < NH; ++ph) {
          raw_load(rq[ph][a], qg + t * DK + DKH * ph + ch0);
          raw_load(rk[ph][a], kg + t * DK + DKH * ph + ch0);
          raw_load(rg[ph][a], gg + t * DK + DKH * ph + ch0);
        }
        raw_load(rv[a], vg + t * DV + vcol0 + vc0);
      } else {
#pragma unroll
        for (int ph = 0; ph < NH; ++ph) {
          raw_zero(rq[ph][a]); raw_zero(rk[ph][a]); raw_zero(rg[ph][a]);
        }
        raw_zero(rv[a]);
      }
    }
  };

  const long len = eos - bos;
  const int nchunks = (int)((len + C - 1) / C);
  if (nchunks > 0) prefetch(bos);

  const int p = w;  // this wave's query sub-chunk in the contractions
  for (int u = 0; u < nchunks; ++u) {
    const long t0 = bos + (long)u * C;
    f32x4 pacc[4];   // transposed score blocks P^T(r, p), summed over the passes
    f32x4 oacc[4];   // O^T of the wave's 16 queries, 4 blocks of 16 columns
#pragma unroll
    for (int r = 0; r < 4; ++r) pacc[r] = oacc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    float vv[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a) raw_unpack<E, 4>(rv[a], vv[a]);

#pragma unroll
    for (int ph = 0; ph < NH; ++ph) {
    // ===================== 1. gating: scan (registers only) =====================
    float loc[4][CPL];      // Gamma relative to the start of the lane's sub-chunk (log2)
    float tot[CPL], Bp[CPL], B4[CPL], s1v[CPL], s2v[CPL];
    {
      float x[4][CPL];
#pragma unroll
      for (int a = 0; a < 4; ++a) raw_unpack<E, CPL>(rg[ph][a], x[a]);
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        float p0 = clamp_gate(x[0][i] * kLog2e);
        float p1 = p0 + clamp_gate(x[1][i] * kLog2e);
        float p2 = p1 + clamp_gate(x[2][i] * kLog2e);
        float p3 = p2 + clamp_gate(x[3][i] * kLog2e);
        // inclusive scan of the lane totals across the 4 lanes of the sub-chunk
        float u4 = p3;
        float t1 = dpp<kRowShr1>(u4);
        u4 += (tg & 3) >= 1 ? t1 : 0.f;
        float t2 = dpp<kRowShr2>(u4);
        u4 += (tg & 3) >= 2 ? t2 : 0.f;
        float ex = dpp<kRowShr1>(u4);
        ex = (tg & 3) >= 1 ? ex : 0.f;        // exclusive prefix inside the sub-chunk
        loc[0][i] = ex + p0;
        loc[1][i] = ex + p1;
        loc[2][i] = ex + p2;
        loc[3][i] = ex + p3;
        const float tt = __int_as_float(
            __builtin_amdgcn_mov_dpp(__float_as_int(u4), kQuadBcast3, 0xF, 0xF, false));
        tot[i] = tt;                               // total of this sub-chunk
        const float a1 = dpp<kRowShr4>(tt);        // total of sub-chunk sub-1 (0 if none)
        const float a2 = dpp<kRowShr8>(tt);        // sub-2
        const float a3 = dpp<kRowShr12>(tt);       // sub-3
        s1v[i] = a1;
        s2v[i] = a2;
        Bp[i] = (a1 + a2) + a3;                    // Gamma at the row before this sub-chunk
        const float bn = Bp[i] + tt;               // Gamma at the sub-chunk's last row
        // Gamma_last: the value computed by sub-chunk 3's lanes, sent to every lane
        const float r4 = dpp<kRowRor4>(bn), r8 = dpp<kRowRor8>(bn), r12 = dpp<kRowRor12>(bn);
        B4[i] = sub == 3 ? bn : sub == 0 ? r4 : sub == 1 ? r8 : r12;
      }
    }
    const int fslot = (u * NH + ph) & 1;
    {
      // path flags of this pass: bit0 = the single-pivot form is unsafe, bit1 = exact
      // diagonal needed
      bool big = false, extreme = false;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        big |= !(fabsf(B4[i]) <= 60.f);
        extreme |= !(fabsf(tot[i]) <= 100.f);
      }
      const unsigned long long bb = __ballot(big), be = __ballot(extreme);
      if (lane == 0) s_flag[fslot][w] = (bb ? 1 : 0) | (be ? 2 : 0);
    }
    __syncthreads();  // (A) previous pass's MFMA reads are done; flags visible
    const int fl = s_flag[fslot][0] | s_flag[fslot][1] | s_flag[fslot][2] | s_flag[fslot][3];
    const bool fast = (fl & 1) == 0;
    const bool exact_diag = (fl & 2) != 0;

    // ===================== 2. gating: operand tiles into LDS =====================
    {
      float qv[4][CPL], kv[4][CPL];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        raw_unpack<E, CPL>(rq[ph][a], qv[a]);
        raw_unpack<E, CPL>(rk[ph][a], kv[a]);
      }
      float fBp[CPL], fKe[CPL], fKP[CPL];
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        fBp[i] = fast_exp2(Bp[i]);
        fKe[i] = fast_exp2(B4[i] - (Bp[i] + tot[i]));
        fKP[i] = fast ? fast_exp2(-(Bp[i] + tot[i])) : 1.f;
      }
      if (exact_diag) {
        // exact diagonal block of this lane's sub-chunk, partial over its channels:
        // d[a][j] = sum_c q_{4tg+a,c} k_{j,c} 2^(Gamma_{4tg+a,c} - Gamma_{j,c}), j in sub-chunk
        float d[4][16];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int j = 0; j < 16; ++j) d[a][j] = 0.f;
#pragma unroll
        for (int src = 0; src < 4; ++src) {   // source lane inside the quad
#pragma unroll
          for (int i = 0; i < CPL; ++i) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const float kj = quad_bcast(kv[b][i], src);
              const float lj = quad_bcast(loc[b][i], src);
              const int j = src * 4 + b;      // key row inside the sub-chunk
#pragma unroll
              for (int a = 0; a < 4; ++a) {
                const int irow = (tg & 3) * 4 + a;
                if (j <= irow) d[a][j] += qv[a][i] * kj * fast_exp2(loc[a][i] - lj);
              }
            }
          }
        }
        // sum over the wave's four lane rows (channel groups), then one partial per wave
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            float x = d[a][j];
            x += __shfl_xor(x, 16);
            x += __shfl_xor(x, 32);
            d[a][j] = x;
          }
        if (gq == 0) {
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int j = 0; j < 16; ++j) s_diag[sub][w][(tg & 3) * 4 + a][j] = d[a][j];
        }
      }
      // S_prev rows of this pass (its inter-term operand) as SBT[col][channel]
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        store4<E>(s_sb + (cb * 16 + m) * PQ + w * WCH + gq * 4, sacc[ph][cb][0], sacc[ph][cb][1],
                  sacc[ph][cb][2], sacc[ph][cb][3]);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int row = 4 * tg + a;
        float qh[CPL], qe[CPL], kt[CPL], kp[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          qh[i] = qv[a][i] * fast_exp2(loc[a][i]);              // Q 2^(Gamma - B_p)
          kt[i] = kv[a][i] * fast_exp2(tot[i] - loc[a][i]);     // K 2^(B_{p+1} - Gamma)
          qe[i] = qh[i] * fBp[i];                               // Q 2^Gamma
          kp[i] = kt[i] * fKP[i];                               // fast: K 2^-Gamma
          kv[a][i] = kt[i] * fKe[i];                            // K 2^(Gamma_last - Gamma)
        }
        lds_store_n<E, CPL>(s_qe + row * PQ + ch0, qe);
        lds_store_n<E, CPL>(s_kp + row * PQ + ch0, kp);
        if (!fast) {
          const int prow = (tg & 3) * 4 + a;  // row inside the sub-chunk
          const int base = sub * (sub + 1) / 2;
          float tmp[CPL];
          // diagonal block (sub, sub): factor 2^(B_p - B_{p+1}) = 2^-tot
#pragma unroll
          for (int i = 0; i < CPL; ++i) tmp[i] = qh[i] * fast_exp2(-tot[i]);
          lds_store_n<E, CPL>(s_qp + ((base + sub) * 16 + prow) * PQ + ch0, tmp);
          if (sub >= 1) lds_store_n<E, CPL>(s_qp + ((base + sub - 1) * 16 + prow) * PQ + ch0, qh);
          if (sub >= 2) {
#pragma unroll
            for (int i = 0; i < CPL; ++i) tmp[i] = qh[i] * fast_exp2(s1v[i]);
            lds_store_n<E, CPL>(s_qp + ((base + sub - 2) * 16 + prow) * PQ + ch0, tmp);
          }
          if (sub >= 3) {
#pragma unroll
            for (int i = 0; i < CPL; ++i) tmp[i] = qh[i] * fast_exp2(s1v[i] + s2v[i]);
            lds_store_n<E, CPL>(s_qp + ((base + sub - 3) * 16 + prow) * PQ + ch0, tmp);
          }
        }
      }
      // K 2^(Gamma_last - Gamma) as KT[channel][token]
#pragma unroll
      for (int i = 0; i < CPL; ++i)
        store4<E>(s_kt + (ch0 + i) * PT + 4 * tg, kv[0][i], kv[1][i], kv[2][i], kv[3][i]);
      // V as VT[column][token], once per chunk (no later pass writes it)
      if (ph == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          store4<E>(s_vt + (vc0 + c) * PT + 4 * tg, vv[0][c], vv[1][c], vv[2][c], vv[3][c]);
      }
      if (tg == 0) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) s_dec[ch0 + i] = fast_exp2(B4[i]);
      }
    }
    // next chunk's inputs are in flight during the last pass's contractions
    if (ph == NH - 1 && u + 1 < nchunks) prefetch(t0 + C);
    __syncthreads();  // (B) operand tiles complete

    // ===================== 3. contractions on MFMA =====================
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r <= p) {
        const S* bsrc = fast ? s_qe + (16 * p + m) * PQ
                             : s_qp + ((p * (p + 1) / 2 + r) * 16 + m) * PQ;
        const S* asrc = s_kp + (16 * r + m) * PQ;
        if (!(r == p && exact_diag)) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            Frag<E> fa, fb;
            frag_ld8(fa, asrc + ks * 32 + gq * 8);
            frag_ld8(fb, bsrc + ks * 32 + gq * 8);
            mma(pacc[r], fa, fb);
          }
        } else {
          // exact diagonal: the four per-wave channel partials, summed in a fixed order
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int j = gq * 4 + s;
            pacc[r][s] += ((s_diag[p][0][m][j] + s_diag[p][1][m][j]) + s_diag[p][2][m][j]) +
                          s_diag[p][3][m][j];
          }
        }
      }
    }
    // O^T += S_prev^T (Q 2^Gamma)^T over this pass's channels
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      Frag<E> fb;
      frag_ld8(fb, s_qe + (16 * p + m) * PQ + ks * 32 + gq * 8);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        Frag<E> fa;
        frag_ld8(fa, s_sb + (cb * 16 + m) * PQ + ks * 32 + gq * 8);
        mma(oacc[cb], fa, fb);
      }
    }
    if (ph == NH - 1) {
      // causal mask of the diagonal block (key j after query i), then
      // O^T += V^T P^T over keys 32ks..32ks+31 (score blocks 2ks, 2ks+1)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (gq * 4 + s > m) pacc[p][s] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (2 * ks <= p) {
          float pv[8] = {pacc[2 * ks][0],     pacc[2 * ks][1],     pacc[2 * ks][2],
                         pacc[2 * ks][3],     pacc[2 * ks + 1][0], pacc[2 * ks + 1][1],
                         pacc[2 * ks + 1][2], pacc[2 * ks + 1][3]};
          Frag<E> fb;
          frag_from_f32(fb, pv);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            Frag<E> fa;
            const S* vrow = s_vt + (cb * 16 + m) * PT + ks * 32 + gq * 4;
            frag_ld4x2(fa, vrow, vrow + 16);
            mma(oacc[cb], fa, fb);
          }
        }
      }
      // store the wave's 16 output rows: lane holds token 16p+m, columns 16cb+4gq..+3
      const long t = t0 + 16 * p + m;
      if (t < eos) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          store4<E>(og + t * DV + vcol0 + cb * 16 + gq * 4, oacc[cb][0], oacc[cb][1],
                    oacc[cb][2], oacc[cb][3]);
      }
    }
    // state rows of this pass: S = diag(2^Gamma_last) S + (K 2^(Gamma_last - Gamma))^T V
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float f = s_dec[w * WCH + gq * 4 + s];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) sacc[ph][cb][s] *= f;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      Frag<E> fa;
      frag_ld8(fa, s_kt + (w * WCH + m) * PT + ks * 32 + gq * 8);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        Frag<E> fb;
        frag_ld8(fb, s_vt + (cb * 16 + m) * PT + ks * 32 + gq * 8);
        mma(sacc[ph][cb], fa, fb);
      }
    }
    }   // passes
  }

  if (prm.sT) {
#pragma unroll
    for (int ph = 0; ph < NH; ++ph)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int c = DKH * ph + w * WCH + gq * 4 + s;
          prm.sT[sbase + (long)c * DV + vcol0 + cb * 16 + m] = sacc[ph][cb][s];
        }
  }
}

template <int DK, typename E>
static int launch(const ChunkParams& prm, int nblocks, hipStream_t stream) {
  hipLaunchKernelGGL((chunk_fwd_kernel<DK, E>), dim3(nblocks), dim3(256), 0, stream, prm);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_chunk_fwd(const ChunkParams& prm, int dk, int dtype, int nblocks, hipStream_t stream) {
  // bf16: the pipelined producer/consumer kernel; fp32: the single-phase kernel above
  if (dtype == 0) return launch_chunk_fwd_pipe(prm, dk, false, nblocks, stream);
  if (dtype == 1 && dk == 64) return launch<64, F32>(prm, nblocks, stream);
  if (dtype == 1 && dk == 128) return launch<128, F32>(prm, nblocks, stream);
  return -2;
}

}  // namespace gla
