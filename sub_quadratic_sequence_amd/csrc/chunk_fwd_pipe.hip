// Pipelined chunkwise GLA forward for gfx950 (MI355X), bf16 inputs, fp32 state.
//
// Same mathematics as chunk_fwd.hip (the chunk form of the page "Gated Linear
// Attention (GLA): Mathematical Foundations ...", section "Mathematical
// Formulation of Chunk Computations"), organised so that the gating work and
// the matrix-core work of consecutive chunks overlap:
//
//  * one workgroup = 8 waves per (sequence, head, slice of d_v): 64 columns,
//    or 128 when the batch has enough units to fill the device with those
//    (NT = 2: the gating of q and k and the score blocks then serve twice the
//    columns); waves 0-3 are producers, waves 4-7 consumers, one of each per
//    SIMD.
//  * producers turn chunk u+1's q, k, g, v into MFMA operand tiles in one LDS
//    buffer while consumers run chunk u's contractions from the other buffer;
//    a single workgroup barrier per chunk swaps them.
//  * producer wave w owns key channels [w DK/4, (w+1) DK/4) of all 64 tokens:
//    lane (tg, gq) holds tokens 4tg..4tg+3 x DK/16 channels, so the log2-gate
//    cumulative sum is a serial sum over 4 tokens plus a 16-lane DPP scan.
//  * consumer wave c owns state columns [16c, 16c+16) of each 64-column half
//    of the slice (all d_k rows) in MFMA accumulators and computes the
//    transposed output tile O^T for those columns and all 64 queries.  The state rows are assigned to accumulator
//    rows so that a lane's accumulator values for a 32-channel step are
//    exactly the 8 contiguous channels its operand fragments use: the
//    inter-chunk term takes S straight from the accumulators as an MFMA
//    operand, without an LDS round trip.
//
// Numerics (decided per chunk and per producer wave, i.e. per 32-channel
// slice, without cross-wave synchronisation):
//  * fast slice (|Gamma_last| <= 60 in log2 units for all its channels):
//    query operand Q 2^Gamma, key operand K 2^-Gamma, state keys K 2^-Gamma
//    with S <- 2^Gamma_last (S + KT^T V).
//  * safe slice: 16-token sub-chunk pivots B_p: query operand
//    Q 2^(Gamma - B_p) (<= |Q|), key operand K 2^(B_{r+1} - Gamma) (<= |K|),
//    per-(p, r) channel factors 2^(B_p - B_{r+1}) applied by the consumer,
//    state keys K 2^(Gamma_last - Gamma) with S <- 2^Gamma_last S + KT^T V.
//  * extreme slice (a 16-token decay beyond 2^100 in one of its channels): the
//    diagonal 16x16 score blocks of that slice are summed element by element
//    by the producer, exp2 of every gate difference, and added by consumers.
#include <type_traits>

#include "gla_device.h"
#include "gla_kernels.h"

namespace gla {

namespace pipe {

constexpr int C = 64;
constexpr float kFastLimit = 60.f;
constexpr float kExtremeLimit = 100.f;
constexpr int kBufferFlags = 0x00020000;   // gfx9 buffer descriptor word 3: raw 32-bit dwords

// LDS tile layouts.  Rows are stored densely and the 16-byte units of a row
// are permuted by XOR with a linear function of the row index, so that both
// the producers' row-wise writes and the consumers' MFMA fragment reads reach
// all LDS banks without conflicts (the maps were chosen by measuring every
// access pattern of this kernel on gfx950).  A linear map lets an address
// split into a per-lane part and a compile-time part: swz(a ^ b) =
// swz(a) ^ swz(b) for row bits that do not overlap.
//
// [token][channel] tiles (query / key operands), DK = 128: 64 rows of 256 B,
// unit u of row r at ((u ^ tok_swz(r)) & 15).  DK = 64 uses 16-byte padded
// rows instead.
__device__ __forceinline__ constexpr int tok_swz(int r) {
  return ((r & 1) ? 2 : 0) ^ ((r & 2) ? 1 : 0) ^ ((r & 4) ? 6 : 0) ^ ((r & 8) ? 15 : 0) ^
         ((r & 16) ? 13 : 0) ^ ((r & 32) ? 10 : 0);
}
// [channel | column][token] tiles (state keys, values): rows of 64 tokens =
// 128 B, 16-byte unit u of row r at ((u ^ tr_swz(r)) & 7).
__device__ __forceinline__ constexpr int tr_swz(int r) {
  return ((r & 1) ? 5 : 0) ^ ((r & 2) ? 1 : 0) ^ ((r & 4) ? 7 : 0) ^ ((r & 8) ? 3 : 0) ^
         ((r & 16) ? 6 : 0) ^ ((r & 64) ? 3 : 0);
}

template <int DK>
struct TokTile {
  static constexpr bool kSwz = DK == 128;
  static constexpr int kPitch = kSwz ? DK : DK + 8;   // elements per row
  // element offset of 8-byte half `h` of 16-byte unit u in row r, with the row's
  // swizzle given separately (sw = tok_swz(r) or its split parts XORed)
  __device__ static __forceinline__ int off(int r, int u, int sw, int h = 0) {
    return r * kPitch + (kSwz ? ((u ^ sw) & 15) : u) * 8 + h * 4;
  }
  __device__ static __forceinline__ int swz(int r) { return kSwz ? tok_swz(r) : 0; }
};
constexpr int TRP = C;   // [channel | column][token] row pitch (elements)
__device__ __forceinline__ int tr_off(int r, int u, int sw, int h = 0) {
  return r * TRP + ((u ^ sw) & 7) * 8 + h * 4;
}

template <int DK, int NT>
struct alignas(256) Buf {
  static constexpr int PQ = TokTile<DK>::kPitch;
  static constexpr int DVT = 64 * NT;   // columns of the slice
  unsigned short q[C * PQ];        // query operand  [token][channel]
  unsigned short k[C * PQ];        // key operand    [token][channel]
  unsigned short kt[DK * TRP];     // state keys     [channel][token]
  unsigned short vt[DVT * TRP];    // values         [column][token]
  unsigned short diag[4][4][16][16];  // exact diagonal partials [slice][sub-chunk][i][j]
  float w[7][DK];      // per-channel pair factors: 0-3 diagonal of sub-chunk p, 4 (2,0), 5 (3,1), 6 (3,0)
  float bq[4][DK];     // inter-term factor per query sub-chunk
  float pre[DK];       // S <- pre * S before the state update
  float post[DK];      // S <- post * S after it
  int flag[4];         // per producer wave: bit0 safe, bit1 extreme
};

// Workgroup barrier that orders LDS only: it waits for this wave's LDS
// operations but not for its outstanding global loads, so prefetches stay in
// flight across it (a __syncthreads() fence would drain them every chunk).
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// N (4 or 8) consecutive floats to 16-byte aligned shared memory.
template <int N>
__device__ __forceinline__ void store_f32(float* p, const float* x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  if constexpr (N == 8) *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

// Hides x's value from the optimiser at this point, so that addresses derived
// from it are recomputed inside the chunk loop (1 VALU op per LDS access)
// instead of being hoisted into dozens of live registers.
__device__ __forceinline__ void launder(int& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void launder(unsigned& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void launder(float& x) { asm volatile("" : "+v"(x)); }

// x from lane QP-permuted inside each quad of lanes (DPP quad_perm control QP)
template <int QP>
__device__ __forceinline__ float quad_perm(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), QP, 0xF, 0xF, false));
}

// consumer state-row map: accumulator tile rb, row m -> key channel
__device__ __forceinline__ int srow(int rb, int m) {
  return 32 * (rb >> 1) + 8 * (m >> 2) + 4 * (rb & 1) + (m & 3);
}

}  // namespace pipe

// MODE kFull: the forward pass (outputs, and the final state of unsplit sequences).
// MODE kFullStates: kFull on 64-column slices that also writes the bf16 state
// entering every chunk, as kChunkStates does.
// MODE kChunkStates: no outputs; the state entering every chunk, in bf16, to
// prm.hs (the backward pass's recomputed states).
// MODE kSegGrad: the state-gradient pass of the backward's sequence split (k and v
// hold q and dO): chunks from last to first, B <- 2^Gamma_last B + (q 2^Gamma)^T dO
// from B = 0 over segments 1 .. nseg-1, to seg_state, with the segment's decay.
// MODE kStateOnly: the state a segment reaches from S = 0 and the segment's total
// gate decay, for the sequence split (no queries read, no outputs written).
template <int DK, int MODE, int NT>
__global__ __launch_bounds__(512, 1) void chunk_fwd_pipe_kernel(ChunkParams prm) {
  using namespace pipe;
  constexpr bool FULL = MODE == kFull || MODE == kFullStates;
  constexpr bool STATES = MODE == kChunkStates;
  constexpr bool REV = MODE == kSegGrad;
  static_assert(!(STATES || MODE == kFullStates) || NT == 1, "chunk states come from 64-column slices");
  static_assert(!REV || NT == 1, "the gradient pass runs on 64-column slices");
  using BufT = Buf<DK, NT>;
  constexpr int DVT = BufT::DVT;
  constexpr int PQ = BufT::PQ;
  constexpr int CPL = DK / 16;   // producer: channels per lane
  constexpr int WCH = DK / 4;    // producer: channels per wave
  constexpr int KS = DK / 32;    // 32-channel contraction steps
  constexpr int NRB = DK / 16;   // consumer: 16-row state tiles
  constexpr int NWR = CPL / 2;   // 32-bit words per lane per token (q, k, g)

  __shared__ __attribute__((aligned(256))) BufT bufs[2];
  // outputs of the 64-column full pass go out through LDS, so that every global
  // store instruction writes whole 128-byte rows: chunk u's [token][column] bf16
  // tile in ostage[u & 1], its 8-byte units XOR-permuted by the row
  constexpr bool OSTAGE = FULL && NT == 1;
  __shared__ __attribute__((aligned(256))) unsigned short ostage[OSTAGE ? 2 : 1][OSTAGE ? C * 64 : 4];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, m = lane & 15, gq = lane >> 4;
  const bool producer = wave < 4;

  // ---- work item ------------------------------------------------------------------
  const int nblk = gridDim.x;
  const int bid = blockIdx.x;
  int item, vt, n, h, seg;   // item = (unit, segment), unit = (sequence n, head h)
  if (prm.sort_units) {
    // Packed sequences of unequal lengths: work items of the longest sequences
    // are dispatched first (all slices of a unit on one XCD: blocks 8s + x),
    // so the longest ones do not start last.  Every workgroup ranks the
    // lengths the same way (ties by index).
    __shared__ int order[kMaxSortSeqs];
    if (wave == 0 && lane < prm.nseq) {
      const int l0 = prm.cu[lane + 1] - prm.cu[lane];
      int rank = 0;
      for (int j = 0; j < prm.nseq; ++j) {
        const int lj = prm.cu[j + 1] - prm.cu[j];
        rank += (lj > l0) || (lj == l0 && j < lane);
      }
      order[rank] = lane;
    }
    __syncthreads();
    const int x = bid & 7, sl = bid >> 3;
    const int r = x + 8 * (sl / prm.nvt);   // unit rank, longest first
    vt = sl - (sl / prm.nvt) * prm.nvt;
    n = order[r / prm.H];
    h = r - (r / prm.H) * prm.H;
    seg = 0;
    item = n * prm.H + h;
  } else {
    const int lin = prm.xcd_remap ? (bid & 7) * (nblk >> 3) + (bid >> 3) : bid;
    item = lin / prm.nvt;
    vt = lin - item * prm.nvt;
    const int nsg = REV ? prm.nseg - 1 : prm.nseg;   // the gradient pass skips segment 0
    const int u0 = item / nsg;
    seg = item - u0 * nsg + (REV ? 1 : 0);
    item = u0 * prm.nseg + seg;
    n = u0 / prm.H;
    h = u0 - n * prm.H;
  }
  const int unit = n * prm.H + h;
  long bos, eos, rowbase;
  if (prm.cu) {
    bos = prm.cu[n];
    eos = prm.cu[n + 1];
    rowbase = (long)h * prm.T;
  } else {
    bos = (long)seg * prm.seg_len;
    eos = bos + prm.seg_len < prm.T ? bos + prm.seg_len : prm.T;
    rowbase = ((long)n * prm.H + h) * prm.T;
  }
  const int DV = prm.DV;
  const int vcol0 = vt * DVT;
  const int nch = (int)((eos - bos + C - 1) / C);
  // state in and out of this work item ([DK][DV] fp32, this slice's columns used)
  const float* s_in;
  float* s_out;
  if constexpr (STATES) {
    s_in = prm.s0 ? prm.s0 + (long)unit * DK * DV : nullptr;
    s_out = nullptr;
  } else if constexpr (!FULL) {
    s_in = nullptr;
    s_out = prm.seg_state + (long)item * DK * DV;
  } else if (prm.nseg > 1) {
    s_in = prm.seg_state + (long)item * DK * DV;   // the segment's incoming state
    s_out = nullptr;
  } else {
    s_in = prm.s0 ? prm.s0 + (long)unit * DK * DV : nullptr;
    s_out = prm.sT ? prm.sT + (long)unit * DK * DV : nullptr;
  }

  if (producer) {
    // =========================== producer waves ===========================
    // Lane (tg, gq) of producer wave w holds tokens 4tg..4tg+3 x key channels
    // w*WCH + gq*CPL .. + CPL: the gate cumsum is a serial sum over 4 tokens
    // plus a 16-lane DPP scan.  Each group of raw registers is reloaded with
    // the next chunk's data as soon as this chunk no longer needs it: v after
    // the value tile is written, g after the gate scan, q and k at the end.
    const int w = wave;
    const int tg = m;                      // tokens 4tg..4tg+3
    const int ch0 = w * WCH + gq * CPL;    // first channel of this lane
    const int sub = tg >> 2;               // 16-token sub-chunk
    // V is loaded and written in its own lane order: lane (tv, gv) = (lane / 4, lane % 4)
    // holds tokens 4tv..4tv+3 of columns vc0..vc0+3, so that four consecutive lanes
    // read one row's 32 bytes (the memory pipeline groups consecutive lanes)
    const int tv = lane >> 2;
    const int vc0 = w * 16 + (lane & 3) * 4;   // first of 4 V columns (of each 64-column half)
    // Raw buffer loads over the sequence's rows: a read past its last row
    // returns zeros (the buffer's record count ends there), which is exactly
    // the padding of a partial last chunk (q = k = v = 0, log-gate 0).  Offsets
    // are byte offsets held whole in the VGPR operand.
    const long r0 = rowbase + bos;
    const int qk_rec = (int)(unsigned)((eos - bos) * DK * 2);   // < 2^32 (host-checked sizes)
    const int v_rec = (int)(unsigned)((eos - bos) * DV * 2);
    const __amdgpu_buffer_rsrc_t rs_q = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(static_cast<const void*>(static_cast<const unsigned short*>(prm.q) + r0 * DK)),
        (short)0, qk_rec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rs_k = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(static_cast<const void*>(static_cast<const unsigned short*>(prm.k) + r0 * DK)),
        (short)0, qk_rec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rs_g = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(static_cast<const void*>(static_cast<const unsigned short*>(prm.g) + r0 * DK)),
        (short)0, qk_rec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rs_v = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(static_cast<const void*>(static_cast<const unsigned short*>(prm.v) + r0 * DV)),
        (short)0, v_rec, kBufferFlags);
    const unsigned qk_lane = ((4 * tg) * DK + ch0) * 2u;          // token 4tg, channel ch0
    const unsigned v_lane = ((4 * tv) * DV + vcol0 + vc0) * 2u;   // token 4tv, column vcol0 + vc0

    unsigned rq[4][NWR], rk[4][NWR], rg[4][NWR], rv[NT][4][2];

    auto ld = [&](unsigned (&r)[NWR], __amdgpu_buffer_rsrc_t rs, unsigned off) __attribute__((always_inline)) {
      if constexpr (NWR == 4) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
        r[0] = x[0]; r[1] = x[1]; r[2] = x[2]; r[3] = x[3];
      } else {
        const auto x = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, 0);
        r[0] = x[0]; r[1] = x[1];
      }
    };
    auto st = [&](unsigned short* p, const unsigned (&r)[NWR]) __attribute__((always_inline)) {
      if constexpr (NWR == 4)
        *reinterpret_cast<uint4*>(p) = uint4{r[0], r[1], r[2], r[3]};
      else
        *reinterpret_cast<uint2*>(p) = uint2{r[0], r[1]};
    };
    auto load_v = [&](int u) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const auto x = __builtin_amdgcn_raw_buffer_load_b64(
              rs_v, (int)(v_lane + 128u * t + (unsigned)(u * C + a) * DV * 2u), 0, 0);
          rv[t][a][0] = x[0]; rv[t][a][1] = x[1];
        }
    };
    auto load_g = [&](int u) __attribute__((always_inline)) {
#pragma unroll
      for (int a = 0; a < 4; ++a) ld(rg[a], rs_g, qk_lane + (unsigned)(u * C + a) * DK * 2u);
    };
    auto load_qk = [&](int u) __attribute__((always_inline)) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        if constexpr (FULL) ld(rq[a], rs_q, qk_lane + (unsigned)(u * C + a) * DK * 2u);
        ld(rk[a], rs_k, qk_lane + (unsigned)(u * C + a) * DK * 2u);
      }
    };
    // bf16 element i (0..CPL-1) of a packed row fragment
    auto el = [&](const unsigned (&r)[NWR], int i) __attribute__((always_inline)) -> float {
      return (i & 1) ? __uint_as_float(r[i >> 1] & 0xffff0000u) : __uint_as_float(r[i >> 1] << 16);
    };
    // This lane's slots, as byte offsets inside a buffer (lane part XOR a
    // compile-time part, plus a compile-time row offset, as for the consumers):
    //  * token a (row 4tg+a) of a [token][channel] operand tile: 16-byte unit
    //    ch0 / 8 (DK = 128) or the 8-byte half of it (DK = 64);
    //  * channel ch0 + i (state keys, tokens 4tg..4tg+3) / column vc0 + c (values,
    //    tokens 4tv..4tv+3) of a [channel | column][token] tile.
    constexpr unsigned kQ = offsetof(BufT, q), kK = offsetof(BufT, k), kKT = offsetof(BufT, kt),
                       kVT = offsetof(BufT, vt);
    const unsigned lp_tok =
        TokTile<DK>::kSwz
            ? (unsigned)(4 * tg * 256 + ((((ch0 >> 3) ^ TokTile<DK>::swz(4 * tg)) & 15) << 4) + ((ch0 >> 2) & 1) * 8)
            : (unsigned)(4 * tg * TokTile<DK>::kPitch * 2 + ch0 * 2);
    const unsigned lp_kt = (unsigned)(ch0 * 128 + ((((tg >> 1) ^ tr_swz(ch0)) & 7) << 4) + (tg & 1) * 8);
    const unsigned lp_vt = (unsigned)(vc0 * 128 + ((((tv >> 1) ^ tr_swz(vc0)) & 7) << 4) + (tv & 1) * 8);
    char* const lds = reinterpret_cast<char*>(bufs);
    unsigned b_tok = 0, b_kt = 0, b_vt = 0;   // this chunk's buffer plus the lane parts
    auto slot = [&](unsigned tile, int a) __attribute__((always_inline)) -> unsigned short* {
      const unsigned o = TokTile<DK>::kSwz ? (b_tok ^ ((unsigned)tok_swz(a) << 4)) + a * 256
                                           : b_tok + a * TokTile<DK>::kPitch * 2;
      return reinterpret_cast<unsigned short*>(lds + o + tile);
    };
    auto kt_slot = [&](int i) __attribute__((always_inline)) -> unsigned short* {
      return reinterpret_cast<unsigned short*>(lds + (b_kt ^ ((unsigned)tr_swz(i) << 4)) + i * 128);
    };
    auto vt_slot = [&](int c) __attribute__((always_inline)) -> unsigned short* {
      return reinterpret_cast<unsigned short*>(lds + (b_vt ^ ((unsigned)tr_swz(c) << 4)) + c * 128);
    };

    // which LDS buffers hold all-ones safe-path factors for this wave's slice
    int ones = 0;
    // state-only pass: the segment's log2 gate total of this lane's channels (its
    // tg == 15 lanes hold the chunk-last-row values)
    float dsum[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) dsum[i] = 0.f;
    // produce chunk uc into B = bufs[bi] and start loading chunk un (a valid chunk index)
    auto produce = [&](BufT& B, int bi, int un) __attribute__((always_inline)) {
      const unsigned bb = (unsigned)(reinterpret_cast<char*>(&B) - lds);
      b_tok = lp_tok + bb;
      b_kt = lp_kt + bb + kKT;
      b_vt = lp_vt + bb + kVT;
      launder(b_tok);
      launder(b_kt);
      launder(b_vt);
      // V as [column][token]: pair tokens (a, a+1) of one column in one word
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int wi = c >> 1;
          const unsigned sel = (c & 1) ? 0x07060302u : 0x05040100u;
          const unsigned lo = __builtin_amdgcn_perm(rv[t][1][wi], rv[t][0][wi], sel);
          const unsigned hi = __builtin_amdgcn_perm(rv[t][3][wi], rv[t][2][wi], sel);
          *reinterpret_cast<uint2*>(vt_slot(64 * t + c)) = uint2{lo, hi};
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      load_v(un);
      if constexpr (REV) {
        // Gamma from gates floored at -256 (log2), so that an alpha = 0 gate
        // cannot produce inf - inf; the state keys q 2^Gamma never exceed |q|,
        // and B <- 2^Gamma_last B + KT^T dO (pre = 2^Gamma_last, post = 1)
        float gf[4][CPL], tot[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const float y = fmaxf(el(rg[a], i) * kLog2e, -256.f);
            gf[a][i] = a ? gf[a - 1][i] + y : y;
          }
          float x = gf[3][i];
          x += dpp<kRowShr1>(x);
          x += dpp<kRowShr2>(x);
          x += dpp<kRowShr4>(x);
          x += dpp<kRowShr8>(x);
          const float ex = x - gf[3][i];
#pragma unroll
          for (int a = 0; a < 4; ++a) gf[a][i] += ex;   // Gamma of token 4tg + a
          tot[i] = x;                                     // the chunk's total at tg == 15
        }
        __builtin_amdgcn_sched_barrier(0);
        load_g(un);
        float kte[4][CPL];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int i = 0; i < CPL; ++i) kte[a][i] = el(rk[a], i) * fast_exp2(gf[a][i]);
#pragma unroll
        for (int i = 0; i < CPL; ++i)
          store4<BF16>(kt_slot(i), kte[0][i], kte[1][i], kte[2][i], kte[3][i]);
        if (tg == 15) {
          float e[CPL], one[CPL];
#pragma unroll
          for (int i = 0; i < CPL; ++i) {
            e[i] = fast_exp2(tot[i]);
            one[i] = 1.f;
            dsum[i] += tot[i];
          }
          store_f32<CPL>(&B.pre[ch0], e);
          store_f32<CPL>(&B.post[ch0], one);
        }
        if (lane == 0) B.flag[w] = 1;
      } else {
        // log2 gates: pp = inclusive prefix over this lane's 4 tokens, inc =
        // inclusive prefix over the chunk at this lane's last token (a 16-lane
        // DPP scan of the lane totals).  Gates are <= 0, so |Gamma| is largest
        // at the chunk's last row; the chunk is a fast one for this wave when
        // every |Gamma| of its slice stays within 2^kFastLimit.  A -inf gate
        // (alpha = 0) makes Gamma infinite and the chunk a safe one.
        float pp[4][CPL], inc[CPL];
        float mx = 0.f;
  #pragma unroll
        for (int i = 0; i < CPL; ++i) {
          pp[0][i] = el(rg[0], i) * kLog2e;
  #pragma unroll
          for (int a = 1; a < 4; ++a) pp[a][i] = fmaf(el(rg[a], i), kLog2e, pp[a - 1][i]);
          float x = pp[3][i];
          x += dpp<kRowShr1>(x);
          x += dpp<kRowShr2>(x);
          x += dpp<kRowShr4>(x);
          x += dpp<kRowShr8>(x);
          inc[i] = x;
          mx = fmaxf(mx, fabsf(x));
        }
        const bool fastw = __ballot(!(mx <= kFastLimit)) == 0ull;
        if (!fastw) {
          // the safe path works from gates floored at -256 (log2), so that an
          // alpha = 0 gate cannot produce inf - inf (laundering keeps the
          // compiler from speculating this rare work into the fast path)
  #pragma unroll
          for (int a = 0; a < 4; ++a)
  #pragma unroll
            for (int j = 0; j < NWR; ++j) launder(rg[a][j]);
  #pragma unroll
          for (int i = 0; i < CPL; ++i) {
  #pragma unroll
            for (int a = 0; a < 4; ++a) {
              const float y = fmaxf(el(rg[a], i) * kLog2e, -256.f);
              pp[a][i] = a ? pp[a - 1][i] + y : y;
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        load_g(un);
        if (fastw) {
          // ---- single pivot at the chunk start ----
          float ex[CPL];   // Gamma before this lane's first token
  #pragma unroll
          for (int i = 0; i < CPL; ++i) ex[i] = inc[i] - pp[3][i];
          unsigned kw[4][NWR];   // packed key operand words, token a
  #pragma unroll
          for (int a = 0; a < 4; ++a) {
            float qe[CPL], ke[CPL];
  #pragma unroll
            for (int i = 0; i < CPL; ++i) {
              const float gm = ex[i] + pp[a][i];   // Gamma of token 4tg+a
              if constexpr (FULL) qe[i] = el(rq[a], i) * fast_exp2(gm);
              ke[i] = el(rk[a], i) * fast_exp2(-gm);
            }
  #pragma unroll
            for (int j = 0; j < NWR; ++j) kw[a][j] = pack_bf16x2(ke[2 * j], ke[2 * j + 1]);
            if constexpr (FULL) {
              lds_store_n<BF16, CPL>(slot(kQ, a), qe);
              st(slot(kK, a), kw[a]);
            }
          }
          // state keys = the same bf16 values, [channel][token]: channel 2j (2j+1)
          // is the low (high) half of word j of the four token rows
  #pragma unroll
          for (int j = 0; j < NWR; ++j) {
  #pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
              const unsigned sel = hb ? 0x07060302u : 0x05040100u;
              const unsigned lo = __builtin_amdgcn_perm(kw[1][j], kw[0][j], sel);
              const unsigned hi = __builtin_amdgcn_perm(kw[3][j], kw[2][j], sel);
              *reinterpret_cast<uint2*>(kt_slot(2 * j + hb)) = uint2{lo, hi};
            }
          }
          if (tg == 15) {   // this lane's last token is the chunk's last row
            float e[CPL];
  #pragma unroll
            for (int i = 0; i < CPL; ++i) {
              e[i] = fast_exp2(inc[i]);
              if constexpr (!FULL) dsum[i] += inc[i];
            }
            store_f32<CPL>(&B.post[ch0], e);
            // the safe-path factors of this slice are ones; they stay so in this
            // buffer until a safe chunk overwrites them
            if (!(ones & (1 << bi))) {
              float one[CPL];
  #pragma unroll
              for (int i = 0; i < CPL; ++i) one[i] = 1.f;
              store_f32<CPL>(&B.pre[ch0], one);
  #pragma unroll
              for (int p = 0; p < 4; ++p) store_f32<CPL>(&B.bq[p][ch0], one);
  #pragma unroll
              for (int e2 = 0; e2 < 7; ++e2) store_f32<CPL>(&B.w[e2][ch0], one);
            }
          }
          ones |= 1 << bi;
          if (lane == 0) B.flag[w] = 0;
        } else {
          // ---- 16-token sub-chunk pivots ----
          // loc = Gamma relative to the start of the token's sub-chunk, tot = the
          // sub-chunk's total: a 4-lane scan of the lane totals within each quad
  #pragma unroll
          for (int a = 0; a < 4; ++a)
  #pragma unroll
            for (int i = 0; i < CPL; ++i) launder(pp[a][i]);
          float loc[4][CPL], tot[CPL];
          bool ext = false;
  #pragma unroll
          for (int i = 0; i < CPL; ++i) {
            float u4 = pp[3][i];
            const float t1 = dpp<kRowShr1>(u4);
            u4 += (tg & 3) >= 1 ? t1 : 0.f;
            const float t2 = dpp<kRowShr2>(u4);
            u4 += (tg & 3) >= 2 ? t2 : 0.f;
            const float ex = u4 - pp[3][i];
  #pragma unroll
            for (int a = 0; a < 4; ++a) loc[a][i] = ex + pp[a][i];
            const float tt = quad_bcast_c<3>(u4);
            tot[i] = tt;
            ext |= !(fabsf(tt) <= kExtremeLimit);
          }
          const bool extw = __ballot(ext) != 0ull;
          // sub-chunk prefixes: s1 = total of sub-chunk p-1, s2 = of p-2, B_p = Gamma at
          // the row before sub-chunk p, b4 = Gamma at the chunk's last row; identical in
          // the four lanes of a quad, so each lane writes CPL/4 channels' factors
          float fke[CPL];
          {
            float s1v[CPL], s2v[CPL], Bp[CPL], b4[CPL];
  #pragma unroll
            for (int i = 0; i < CPL; ++i) {
              const float tt = tot[i];
              const float a1 = dpp<kRowShr4>(tt), a2 = dpp<kRowShr8>(tt), a3 = dpp<kRowShr12>(tt);
              s1v[i] = a1;
              s2v[i] = a2;
              Bp[i] = (a1 + a2) + a3;
              const float bn = Bp[i] + tt;
              const float r4 = dpp<kRowRor4>(bn), r8 = dpp<kRowRor8>(bn), r12 = dpp<kRowRor12>(bn);
              b4[i] = sub == 3 ? bn : sub == 0 ? r4 : sub == 1 ? r8 : r12;
              fke[i] = fast_exp2(b4[i] - bn);   // 2^(Gamma_last - B_{p+1})
              if constexpr (!FULL) dsum[i] += b4[i];
            }
            constexpr int NPL = CPL / 4;
            const int qd = tg & 3;
            auto pick = [&](const float (&x)[CPL], int j) __attribute__((always_inline)) -> float {
              return qd == 0 ? x[j] : qd == 1 ? x[NPL + j] : qd == 2 ? x[2 * NPL + j] : x[3 * NPL + j];
            };
  #pragma unroll
            for (int j = 0; j < NPL; ++j) {
              const int c = ch0 + qd * NPL + j;
              const float s1 = pick(s1v, j);
              const float ebq = fast_exp2(pick(Bp, j));
              // an extreme slice's diagonal blocks come from the exact partials alone
              const float ew = extw ? 0.f : fast_exp2(-pick(tot, j));
              const float e1 = fast_exp2(s1);
              const float e12 = fast_exp2(s1 + pick(s2v, j));
              const float epre = fast_exp2(pick(b4, j));
              B.bq[sub][c] = ebq;
              B.w[sub][c] = ew;
              if (sub == 2) B.w[4][c] = e1;
              if (sub == 3) {
                B.w[5][c] = e1;
                B.w[6][c] = e12;
              }
              if (sub == 0) {
                B.pre[c] = epre;
                B.post[c] = 1.f;
              }
            }
          }
          if (FULL && extw) {
            // exact diagonal partials, one (row a, key pair jj) at a time: sum over this
            // lane's channels, then over the wave's four lane rows (its whole slice)
  #pragma unroll
            for (int a = 0; a < 4; ++a) {
              const int irow = (tg & 3) * 4 + a;
  #pragma unroll
              for (int jj = 0; jj < 8; ++jj) {
                __builtin_amdgcn_sched_barrier(0);
                float dd[2];
  #pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                  const int j = 2 * jj + h2, src = j >> 2, b = j & 3;
                  float acc = 0.f;
  #pragma unroll
                  for (int i2 = 0; i2 < NWR; ++i2) {
                    const unsigned kw = __builtin_bit_cast(unsigned, quad_bcast(__builtin_bit_cast(float, rk[b][i2]), src));
                    const float l0 = quad_bcast(loc[b][2 * i2], src);
                    const float l1 = quad_bcast(loc[b][2 * i2 + 1], src);
                    acc += el(rq[a], 2 * i2) * __uint_as_float(kw << 16) * fast_exp2(loc[a][2 * i2] - l0);
                    acc += el(rq[a], 2 * i2 + 1) * __uint_as_float(kw & 0xffff0000u) *
                           fast_exp2(loc[a][2 * i2 + 1] - l1);
                  }
                  acc = j <= irow ? acc : 0.f;
                  acc += __shfl_xor(acc, 16);
                  acc += __shfl_xor(acc, 32);
                  dd[h2] = acc;
                }
                if (gq == 0)
                  *reinterpret_cast<unsigned*>(&B.diag[w][sub][irow][2 * jj]) = pack_bf16x2(dd[0], dd[1]);
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          float kte[4][CPL];
  #pragma unroll
          for (int a = 0; a < 4; ++a) {
            float qh[CPL], kt[CPL];
  #pragma unroll
            for (int i = 0; i < CPL; ++i) {
              if constexpr (FULL) qh[i] = el(rq[a], i) * fast_exp2(loc[a][i]);   // Q 2^(Gamma - B_p)
              kt[i] = el(rk[a], i) * fast_exp2(tot[i] - loc[a][i]);   // K 2^(B_{p+1} - Gamma)
              kte[a][i] = kt[i] * fke[i];                          // K 2^(Gamma_last - Gamma)
            }
            if constexpr (FULL) {
              lds_store_n<BF16, CPL>(slot(kQ, a), qh);
              lds_store_n<BF16, CPL>(slot(kK, a), kt);
            }
          }
  #pragma unroll
          for (int i = 0; i < CPL; ++i)
            store4<BF16>(kt_slot(i), kte[0][i], kte[1][i], kte[2][i], kte[3][i]);
          if (lane == 0) B.flag[w] = 1 | (extw ? 2 : 0);
          ones &= ~(1 << bi);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      load_qk(un);
    };

    // step i produces chunk i into bufs[i & 1] while the consumers use chunk i-1;
    // the look-ahead index is clamped, so the last step re-reads the last chunk
    // and no load sits behind a branch
    // chunk processed at step i (the gradient pass walks them from last to first)
    auto ck = [&](int i) __attribute__((always_inline)) { return REV ? nch - 1 - i : i; };
    if (nch > 0) {
      load_v(ck(0));
      load_g(ck(0));
      load_qk(ck(0));
    }
    for (int i = 0; i <= nch; ++i) {
      if (i < nch) produce(bufs[i & 1], i & 1, ck(i + 1 < nch ? i + 1 : i));
      barrier_lds();
    }
    if constexpr (MODE == kStateOnly || REV) {
      // the segment's decay exp(sum of g) per key channel, once per (unit, segment)
      if (vt == 0 && tg == 15) {
        float e[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) e[i] = fast_exp2(dsum[i]);
        float* dst = prm.seg_decay + (long)item * DK + ch0;
#pragma unroll
        for (int i = 0; i < CPL; ++i) dst[i] = e[i];
      }
    }
  } else {
    // =========================== consumer waves ===========================
    const int cw = wave - 4;               // state / output columns 64t + [16cw, 16cw+16)
    const int vrow = cw * 16 + m;          // this lane's row of the values tile (t = 0)
    // Per-lane byte offsets of the operand fragments inside a buffer.  With the
    // swizzled layouts a fragment's offset is (lane part) XOR (compile-time part)
    // plus a compile-time row offset: the XOR touches only bits 4-6 (4-7 for the
    // 256-byte token rows), which the buffer base (a multiple of 256) and the row
    // offsets leave clear, so each read costs one v_xor and an immediate offset.
    constexpr unsigned kQ = offsetof(BufT, q), kK = offsetof(BufT, k), kKT = offsetof(BufT, kt),
                       kVT = offsetof(BufT, vt);
    static_assert(kQ % 256 == 0 && kK % 256 == 0 && kKT % 256 == 0 && kVT % 256 == 0 &&
                  sizeof(BufT) % 256 == 0, "fragment offsets assume 256-byte aligned tiles");
    const unsigned lb_qk = TokTile<DK>::kSwz
                               ? (unsigned)(m * 256 + ((gq ^ TokTile<DK>::swz(m)) << 4))
                               : (unsigned)(m * TokTile<DK>::kPitch * 2 + gq * 16);
    const unsigned lb_kt = (unsigned)(srow(0, m) * 128 + (((gq ^ tr_swz(srow(0, m))) & 7) << 4));
    const unsigned lb_vb = (unsigned)(vrow * 128 + (((gq ^ tr_swz(vrow)) & 7) << 4));
    const unsigned lb_va = (unsigned)(vrow * 128 + ((((gq >> 1) ^ tr_swz(vrow)) & 7) << 4) + (gq & 1) * 8);
    // Row 64t + r of a values tile sits at row r's place XOR (tr_swz(64) << 4),
    // 64 rows (8 KB) further on.
    constexpr unsigned kHalfX = (unsigned)tr_swz(64) << 4, kHalfOff = 64u * 128u;
    unsigned short* og = reinterpret_cast<unsigned short*>(prm.o) + rowbase * DV + vcol0;
    // chunk states (the chunk-state mode, and the full pass that also writes them):
    // this unit's first slot, and the lane's element of a slot for tile 0 (the tile
    // is added per store)
    constexpr bool HS = STATES || MODE == kFullStates;
    unsigned short* hs_unit = nullptr;
    int hs_lane = 0;
    if constexpr (HS) {
      const long slot0 = prm.cu ? (long)h * prm.slots + n + bos / C
                                : (long)h * prm.slots + n + (long)n * prm.T / C;
      hs_unit = prm.hs + slot0 * DK * DV;
      // chunk_state_index(srow(0, 4gq + (m & 3)), 64vt + 16cw + 4(m >> 2)) = tile 4vt + cw,
      // row block 2gq, column group m >> 2, row m & 3; state tile rb adds hs_tile(rb)
      hs_lane = (vt * 4 + cw) * 16 * DK + 128 * gq + 4 * m;
    }
    f32x4 sacc[NT][NRB];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int c = srow(rb, gq * 4 + s);
          sacc[t][rb][s] = s_in ? s_in[(long)c * DV + vcol0 + 64 * t + cw * 16 + m] : 0.f;
        }
    // one chunk of contractions; SAFE / EXT are compile-time so the body is branch-free
    auto consume = [&](const BufT& B, int u, auto safe_tag, auto ext_tag) __attribute__((always_inline)) {
      const unsigned bb = (unsigned)(reinterpret_cast<const char*>(&B) - reinterpret_cast<const char*>(bufs));
      unsigned b_qk = lb_qk + bb, b_kt = lb_kt + bb + kKT, b_vb = lb_vb + bb + kVT, b_va = lb_va + bb + kVT;
      launder(b_qk);
      launder(b_kt);
      launder(b_vb);
      launder(b_va);
      const char* lds = reinterpret_cast<const char*>(bufs);
      // fragment (p, ks) of a [token][channel] tile at byte offset tile_off
      auto tok_frag = [&](Frag<BF16>& f, unsigned tile_off, int p, int ks) __attribute__((always_inline)) {
        unsigned a;
        if constexpr (TokTile<DK>::kSwz)
          a = (b_qk ^ ((unsigned)((4 * ks) ^ tok_swz(16 * p)) << 4)) + tile_off + p * 16 * 256;
        else
          a = b_qk + tile_off + p * 16 * TokTile<DK>::kPitch * 2 + ks * 64;
        f.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(lds + a));
      };      constexpr bool SAFE = decltype(safe_tag)::value;
      constexpr bool EXT = decltype(ext_tag)::value;
      // scaled copy of a query fragment by 8 per-channel factors
      auto scaled = [&](const Frag<BF16>& f, const float* wrow, int ks) __attribute__((always_inline)) {
        const float4 w0 = *reinterpret_cast<const float4*>(wrow + ks * 32 + gq * 8);
        const float4 w1 = *reinterpret_cast<const float4*>(wrow + ks * 32 + gq * 8 + 4);
        const uint4 r = __builtin_bit_cast(uint4, f.v);
        float x[8];
        x[0] = __uint_as_float(r.x << 16) * w0.x; x[1] = __uint_as_float(r.x & 0xffff0000u) * w0.y;
        x[2] = __uint_as_float(r.y << 16) * w0.z; x[3] = __uint_as_float(r.y & 0xffff0000u) * w0.w;
        x[4] = __uint_as_float(r.z << 16) * w1.x; x[5] = __uint_as_float(r.z & 0xffff0000u) * w1.y;
        x[6] = __uint_as_float(r.w << 16) * w1.z; x[7] = __uint_as_float(r.w & 0xffff0000u) * w1.w;
        Frag<BF16> o;
        frag_from_f32(o, x);
        return o;
      };
      if constexpr (FULL) {   // outputs of this chunk (the state-only pass has none)
        // S_prev as the inter term's A operand: slots = channels 32ks+8gq..+7 (see srow)
        Frag<BF16> sa[NT][KS];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const float sv[8] = {sacc[t][2 * ks][0],     sacc[t][2 * ks][1],     sacc[t][2 * ks][2],
                                 sacc[t][2 * ks][3],     sacc[t][2 * ks + 1][0], sacc[t][2 * ks + 1][1],
                                 sacc[t][2 * ks + 1][2], sacc[t][2 * ks + 1][3]};
            frag_from_f32(sa[t][ks], sv);
          }
        // V^T rows of this wave's columns, tokens in the score accumulators' order
        Frag<BF16> va[NT][2];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            // tokens 32ks + 4gq .. +3 and the same 16 tokens later
            const unsigned bt = t ? (b_va ^ kHalfX) + kHalfOff : b_va;
            const uint2 lo = *reinterpret_cast<const uint2*>(lds + (bt ^ ((unsigned)(4 * ks) << 4)));
            const uint2 hi = *reinterpret_cast<const uint2*>(lds + (bt ^ ((unsigned)(4 * ks + 2) << 4)));
            va[t][ks].v = __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
          }
        Frag<BF16> kf[4][KS];   // key fragments of sub-chunk r, loaded when first needed
        f32x4 oacc[1][4];   // NT == 1: outputs stored after the four sub-chunks
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          Frag<BF16> qf[KS];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            tok_frag(kf[p][ks], kK, p, ks);
            tok_frag(qf[ks], kQ, p, ks);
          }
          // scores P^T(r, p) = K_r Q_p^T, r <= p
          f32x4 pacc[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) pacc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int r = 0; r <= p; ++r) {
            const int widx = (p == r) ? p : (p == 2 && r == 0) ? 4 : (p == 3 && r == 1) ? 5 : (p == 3 && r == 0) ? 6 : -1;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              if (SAFE && widx >= 0) {
                const Frag<BF16> b = scaled(qf[ks], B.w[widx], ks);
                mma(pacc[r], kf[r][ks], b);
              } else {
                mma(pacc[r], kf[r][ks], qf[ks]);
              }
            }
          }
          // the inter term does not wait for the scores: its products go into the
          // matrix pipeline while the score results are still on their way
          f32x4 o2[NT];
#pragma unroll
          for (int t = 0; t < NT; ++t) o2[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            if constexpr (SAFE) {
              const Frag<BF16> b = scaled(qf[ks], B.bq[p], ks);
#pragma unroll
              for (int t = 0; t < NT; ++t) mma(o2[t], sa[t][ks], b);
            } else {
#pragma unroll
              for (int t = 0; t < NT; ++t) mma(o2[t], sa[t][ks], qf[ks]);
            }
          }
          if constexpr (EXT) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const int j = gq * 4 + s;
              float e = 0.f;
#pragma unroll
              for (int sl = 0; sl < 4; ++sl)
                e += (B.flag[sl] & 2) ? bf16_bits_to_f32(B.diag[sl][p][m][j]) : 0.f;
              pacc[p][s] += e;
            }
          }
#pragma unroll
          for (int s = 0; s < 4; ++s) pacc[p][s] = (gq * 4 + s > m) ? 0.f : pacc[p][s];  // causal

          // O^T(p) = V^T P^T + S_prev^T (Q 2^Gamma)^T
          f32x4 o1[NT];
#pragma unroll
          for (int t = 0; t < NT; ++t) o1[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; 2 * ks <= p; ++ks) {
            const float pv[8] = {pacc[2 * ks][0],     pacc[2 * ks][1],     pacc[2 * ks][2],
                                 pacc[2 * ks][3],     pacc[2 * ks + 1][0], pacc[2 * ks + 1][1],
                                 pacc[2 * ks + 1][2], pacc[2 * ks + 1][3]};
            Frag<BF16> pb;
            frag_from_f32(pb, pv);
#pragma unroll
            for (int t = 0; t < NT; ++t) mma(o1[t], va[t][ks], pb);
          }
          if constexpr (NT == 1) {
            oacc[0][p] = o1[0] + o2[0];
          } else {   // two slices' accumulators do not fit beside the state: store now
            const long tk = bos + (long)u * C + 16 * p + m;
            if (tk < eos) {
#pragma unroll
              for (int t = 0; t < NT; ++t) {
                const f32x4 x = o1[t] + o2[t];
                store4<BF16>(og + tk * DV + 64 * t + cw * 16 + gq * 4, x[0], x[1], x[2], x[3]);
              }
            }
          }
        }
        if constexpr (NT == 1) {
          // token 16p + m, columns 16cw + 4gq .. +3: 8-byte unit 4cw + gq of the row
          unsigned so = (unsigned)(m * 128 + (((4 * cw + gq) ^ m) << 3));
          launder(so);
          char* const ob = reinterpret_cast<char*>(ostage[u & 1]);
#pragma unroll
          for (int p = 0; p < 4; ++p)
            *reinterpret_cast<uint2*>(ob + so + p * 16 * 128) =
                uint2{pack_bf16x2(oacc[0][p][0], oacc[0][p][1]), pack_bf16x2(oacc[0][p][2], oacc[0][p][3])};
        }
      }

      if constexpr (HS) {
        {
          // the state entering chunk u, bf16, in the chunk_state_index order.  Lane
          // (m = 4a + j, gq) holds rows srow(rb, 4gq + 0..3) of column 16cw + m; a
          // 4 x 4 transpose inside each quad of lanes (two DPP exchange stages)
          // leaves it row srow(rb, 4gq + j) of columns 16cw + 4a .. +3, which are 8
          // contiguous bytes of the slot: 8 eight-byte stores per lane and chunk.
          unsigned short* const hu = hs_unit + (long)u * DK * DV;
          const bool o1 = lane & 1, o2 = lane & 2;
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) {
            float y[4], z[4];
#pragma unroll
            for (int p = 0; p < 2; ++p) {   // lane bit 0 <-> slot bit 0
              const float x0 = sacc[0][rb][2 * p], x1 = sacc[0][rb][2 * p + 1];
              const float r = quad_perm<0xB1>(o1 ? x0 : x1);   // [1, 0, 3, 2]
              y[2 * p] = o1 ? r : x0;
              y[2 * p + 1] = o1 ? x1 : r;
            }
#pragma unroll
            for (int p = 0; p < 2; ++p) {   // lane bit 1 <-> slot bit 1
              const float r = quad_perm<0x4E>(o2 ? y[p] : y[p + 2]);   // [2, 3, 0, 1]
              z[p] = o2 ? r : y[p];
              z[p + 2] = o2 ? y[p + 2] : r;
            }
            // rows srow(rb, .) start at row block 8 (rb >> 1) + (rb & 1) of the tile
            const int hs_tile = 512 * (rb >> 1) + 64 * (rb & 1);
            *reinterpret_cast<uint2*>(hu + hs_lane + hs_tile) =
                uint2{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])};
          }
        }
      }
      // ---- state: S <- post * (pre * S + KT^T V) ----
      // every operand is read first (the output phase's registers are free by now),
      // so the 2 NRB products issue back to back
      Frag<BF16> vb[NT][2], ka[2][NRB];
      float4 fpost[NRB];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const unsigned bt = t ? (b_vb ^ kHalfX) + kHalfOff : b_vb;
          vb[t][ks].v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(lds + (bt ^ ((unsigned)(4 * ks) << 4))));
        }
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const unsigned a = (b_kt ^ ((unsigned)(((4 * ks) ^ tr_swz(srow(rb, 0))) & 7) << 4)) + srow(rb, 0) * 128;
          ka[ks][rb].v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(lds + a));
        }
      }
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) fpost[rb] = *reinterpret_cast<const float4*>(&B.post[srow(rb, gq * 4)]);
      if constexpr (SAFE) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const float4 f = *reinterpret_cast<const float4*>(&B.pre[srow(rb, gq * 4)]);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            sacc[t][rb][0] *= f.x; sacc[t][rb][1] *= f.y; sacc[t][rb][2] *= f.z; sacc[t][rb][3] *= f.w;
          }
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
          for (int t = 0; t < NT; ++t) mma(sacc[t][rb], ka[ks][rb], vb[t][ks]);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const float4 f = fpost[rb];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          sacc[t][rb][0] *= f.x; sacc[t][rb][1] *= f.y; sacc[t][rb][2] *= f.z; sacc[t][rb][3] *= f.w;
        }
      }
    };
    // staged outputs of chunk u: wave cw stores rows 16cw .. 16cw+15, 8 rows of
    // 128 bytes per instruction
    auto flush_out = [&](int u) __attribute__((always_inline)) {
      const char* const ob = reinterpret_cast<const char*>(ostage[u & 1]);
      const int j = lane & 7;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int r = 16 * cw + 8 * hh + (lane >> 3);
        // 8-byte units 2j and 2j + 1 of row r sit in the 16-byte block j ^ ((r & 15) >> 1),
        // in swapped order when r is odd
        const uint4 x = *reinterpret_cast<const uint4*>(ob + r * 128 + ((j ^ ((r & 15) >> 1)) << 4));
        const bool sw = r & 1;
        const uint4 y = sw ? uint4{x.z, x.w, x.x, x.y} : x;
        const long tk = bos + (long)u * C + r;
        if (tk < eos) *reinterpret_cast<uint4*>(og + tk * DV + 8 * j) = y;
      }
    };
    using T_ = std::integral_constant<bool, true>;
    using F_ = std::integral_constant<bool, false>;
    for (int i = 0; i <= nch; ++i) {
      if (i > 0) {
        const int u = i - 1;
        if constexpr (OSTAGE) {
          if (u > 0) flush_out(u - 1);
        }
        const BufT& B = bufs[u & 1];
        const int fl = B.flag[0] | B.flag[1] | B.flag[2] | B.flag[3];
        if (fl == 0)
          consume(B, u, F_{}, F_{});
        else if ((fl & 2) == 0)
          consume(B, u, T_{}, F_{});
        else
          consume(B, u, T_{}, T_{});
      }
      barrier_lds();
    }
    if constexpr (OSTAGE) {
      if (nch > 0) flush_out(nch - 1);
    }
    if (s_out) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int c = srow(rb, gq * 4 + s);
            s_out[(long)c * DV + vcol0 + 64 * t + cw * 16 + m] = sacc[t][rb][s];
          }
    }
  }
}

int launch_chunk_seg_grad(const ChunkParams& prm, int dk, int nblocks, hipStream_t stream) {
  if (prm.dvt != 64 || prm.nvt * 64 != prm.DV || prm.nseg < 2 || prm.cu || prm.sort_units) return -2;
  if (dk == 128)
    hipLaunchKernelGGL((chunk_fwd_pipe_kernel<128, kSegGrad, 1>), dim3(nblocks), dim3(512), 0, stream, prm);
  else if (dk == 64)
    hipLaunchKernelGGL((chunk_fwd_pipe_kernel<64, kSegGrad, 1>), dim3(nblocks), dim3(512), 0, stream, prm);
  else
    return -2;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_chunk_fwd_states(const ChunkParams& prm, int dk, int nblocks, hipStream_t stream) {
  if (prm.dvt != 64 || prm.nvt * 64 != prm.DV || prm.nseg != 1) return -2;
  if (dk == 128)
    hipLaunchKernelGGL((chunk_fwd_pipe_kernel<128, kChunkStates, 1>), dim3(nblocks), dim3(512), 0, stream, prm);
  else if (dk == 64)
    hipLaunchKernelGGL((chunk_fwd_pipe_kernel<64, kChunkStates, 1>), dim3(nblocks), dim3(512), 0, stream, prm);
  else
    return -2;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_chunk_fwd_full_states(const ChunkParams& prm, int dk, int nblocks, hipStream_t stream) {
  if (prm.dvt != 64 || prm.nvt * 64 != prm.DV || prm.nseg != 1) return -2;
  if (dk == 128)
    hipLaunchKernelGGL((chunk_fwd_pipe_kernel<128, kFullStates, 1>), dim3(nblocks), dim3(512), 0, stream, prm);
  else if (dk == 64)
    hipLaunchKernelGGL((chunk_fwd_pipe_kernel<64, kFullStates, 1>), dim3(nblocks), dim3(512), 0, stream, prm);
  else
    return -2;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_chunk_fwd_pipe(const ChunkParams& prm, int dk, bool state_only, int nblocks,
                          hipStream_t stream) {
  // the slice width must tile d_v exactly
  if (prm.dvt * prm.nvt != prm.DV || (prm.dvt != 64 && prm.dvt != 128)) return -2;
  const bool wide = prm.dvt == 128;
#define GLA_PIPE(D, M, N) \
  hipLaunchKernelGGL((chunk_fwd_pipe_kernel<D, M, N>), dim3(nblocks), dim3(512), 0, stream, prm)
  if (dk == 128) {
    if (state_only) {
      if (wide) GLA_PIPE(128, kStateOnly, 2); else GLA_PIPE(128, kStateOnly, 1);
    } else {
      if (wide) GLA_PIPE(128, kFull, 2); else GLA_PIPE(128, kFull, 1);
    }
  } else if (dk == 64) {
    if (state_only) {
      if (wide) GLA_PIPE(64, kStateOnly, 2); else GLA_PIPE(64, kStateOnly, 1);
    } else {
      if (wide) GLA_PIPE(64, kFull, 2); else GLA_PIPE(64, kFull, 1);
    }
  } else {
    return -2;
  }
#undef GLA_PIPE
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gla
