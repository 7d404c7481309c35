// Chunkwise GLA backward pass for gfx950 (MI355X), bf16 inputs, fp32 states.
//
// The gradients of L = sum_t <dO_t, o_t> + <dS_T, S_T> for the recurrence of
// the page "Gated Linear Attention (GLA): Mathematical Foundations ...",
// section "The Gated Recurrent Update" (S_t = diag(alpha_t) S_{t-1} + k_t^T v_t,
// o_t = q_t S_t), organised as that page's section "I/O-Aware Kernel Design in
// FlashLinearAttention" describes the backward kernel: chunk states are
// recomputed in the backward call instead of being kept from the forward.
//
// Kernels of one call:
//  * the forward's pipelined kernel in its chunk-state mode (chunk_fwd_pipe.hip):
//    one pass over each sequence that writes the state at the start of every
//    64-token chunk (bf16, one dk x dv slot per chunk, element order
//    chunk_state_index) into the workspace.
//  * when the sequences are split into segments (few units, long sequences):
//    the same pipelined kernel in its segment-gradient mode, run backwards over
//    each segment but one on q 2^Gamma and dO, gives the state gradient a
//    segment sends to its start from its own outputs (and its total decay); the
//    reverse segment scan turns those into each segment's incoming gradient.
//  * chunk_bwd_kernel: one workgroup (8 waves) per (sequence, head) walks the
//    chunks from last to first.  Per chunk, with 16-token sub-chunks s:
//      - a forward sweep s = 0..3 carries the state H (fp32 MFMA accumulators,
//        from the stored chunk-start state) and produces dq;
//      - a reverse sweep s = 3..0 carries the state gradient B (fp32
//        accumulators, from dS_T at the sequence end) and produces dk, dv, dg.
//    With Gamma the in-chunk cumulative log2 gate, the pivot b_s (middle of
//    the sub-chunk's Gamma range) and Delta = Gamma - b_s:
//      q~ = q 2^Delta, k~ = k 2^-Delta, A = dO V^T, P = q~ k~^T (causal)
//      dq = 2^Delta (A k~ + dO H^^T),  dk = 2^-Delta (A^T q~ + V B^^T),
//      dv = P^T dO + k~ B^,
//    where H^ = 2^(b_s - Gamma_{s-1,last}) H and B^ = 2^(Gamma_{s,last} - b_s) B
//    are the carried states scaled by factors <= 1, and
//      H <- 2^(Gamma_{s,last} - b_s) (H^ + k~^T V),
//      B <- 2^(b_s - Gamma_{s-1,last}) (B^ + q~^T dO).
//    Between two sub-chunks the two factors combine into one, 2^(b_s - b_{s-1}),
//    so the carried states are scaled once per step.
//    The gate gradient is the reverse cumulative sum of q*dq - k*dk inside the
//    chunk, started from sum_n H[c][n] B[c][n] at the chunk's end (the gradient
//    of a log-gate is the state times its gradient summed over columns), so
//    rounding does not accumulate along the sequence.
//  Every factor stays within 2^+-120 as long as no channel decays by more than
//  2^-240 inside one 16-token sub-chunk; beyond that the sub-chunk's pivot is
//  set to NaN and the sequence's gradients come out NaN (a loud failure, not a
//  silent one).
#include "gla_device.h"
#include "gla_kernels.h"

namespace gla {

namespace bwd {

constexpr int C = 64;        // chunk
constexpr int L = 16;        // sub-chunk
constexpr int NS = C / L;    // sub-chunks per chunk
constexpr float kRangeLimit = 240.f;
constexpr int kBufferFlags = 0x00020000;   // gfx9 buffer descriptor word 3: raw 32-bit dwords

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Workgroup barrier ordering LDS only (outstanding global loads stay in flight).
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS tiles.  Rows are 256 bytes (16 units of 16 bytes; a tile of 64 bf16
// columns uses half of each row, the fp32 Delta tile of 128 channels spans two
// 256-byte halves), and unit u of row r is stored at unit u ^ swz(r).  gfx950's
// LDS serves 8-byte and transposing reads 32 consecutive lanes per pass over
// 64 banks, 16-byte reads in passes that pair lane quads of equal parity of
// lane bits 2-4, and 8- and 16-byte writes 16 and 8 consecutive lanes per pass
// over 32 banks (all measured with rocprofv3's SQ_LDS_BANK_CONFLICT).  With
// this swz every access shape of the kernel below is free of bank conflicts:
// 8- and 16-byte fragment reads on 16 consecutive rows, transposing reads on
// 8 rows (4 consecutive rows per 16 lanes, also 8-row strided pairs of the
// state tile), the
// gating writes to rows 4t + a (t = 0..7) and the row-wise copies.  The one
// exception is the state tile's 8-byte writes, 2-way by their lane shape.
// swz is linear over the row bits: for row and unit parts with disjoint bits an
// address is (lane part) ^ cx(compile-time part) + ca(compile-time part).
__host__ __device__ constexpr unsigned swz(unsigned r) {
  return ((r & 1) ? 8u : 0u) ^ ((r & 2) ? 4u : 0u) ^ ((r & 4) ? 2u : 0u) ^ ((r & 8) ? 3u : 0u) ^
         ((r & 16) ? 4u : 0u);
}
// byte offset of byte b of unit u in row r of a tile with RB-byte rows
__host__ __device__ constexpr unsigned toff(unsigned r, unsigned u, unsigned b, unsigned RB = 256) {
  return r * RB + (((u & 15u) ^ swz(r)) << 4) + ((u & ~15u) << 4) + b;
}
// XOR and additive parts of a compile-time row cr and unit cu
__host__ __device__ constexpr unsigned cx(unsigned cr, unsigned cu) { return ((cu & 15u) ^ swz(cr)) << 4; }
__host__ __device__ constexpr unsigned ca(unsigned cr, unsigned cu, unsigned RB = 256) {
  return cr * RB + ((cu & ~15u) << 4);
}

// MFMA operand fragments.  A 16-deep operand gives lane (m = lane % 16,
// grp = lane / 16) four contraction indices 4 grp + 0..3 of row (A) or column
// (B) m; a 32-deep operand gives it 8 grp + 0..7.  Both operands of a product
// are built with the same index map, so the contraction is exact whatever
// order the hardware assigns to the slots.
//  * row fragment: from storage [m][k] (k contiguous), one 8- or 16-byte read;
//  * transposed fragment: from storage [k][m] (m contiguous) with the gfx950
//    transposing read: in each 16-lane group, lane i reads 4 consecutive m of
//    row k0 + 4 grp + i / 4 at m0 + 4 (i % 4) and receives element m0 + i of
//    rows k0 + 4 grp + 0..3.
__device__ __forceinline__ s16x4 tr_read(const unsigned short* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}
// 16-deep contraction on the 16x16x16 bf16 instruction (on gfx950 it issues at
// the rate of the 32-deep one, so it saves no matrix-core time, only the moves
// that would build zero-padded 32-deep operands).  Rule: its accumulator input
// is never a register that a 16x16x32 instruction has just written.  The
// compiler separates that dependence by 0-5 wait states on gfx950, and the
// 16-deep instruction then adds to a stale accumulator (wrong values, no
// fault; with 16 wait states in front of it the results are right).  A sum of
// 32-deep and 16-deep products therefore takes the 16-deep one in a fresh
// accumulator (mma16_add); chains of 16-deep products on one accumulator, with
// VALU scalings between them, are fine.
__device__ __forceinline__ void mma16(f32x4& acc, s16x4 a, s16x4 b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
}
// acc += A B (16-deep) where acc comes from 16x16x32 products
__device__ __forceinline__ void mma16_add(f32x4& acc, s16x4 a, s16x4 b) {
  f32x4 t = {0.f, 0.f, 0.f, 0.f};
  mma16(t, a, b);
  acc += t;
}
__device__ __forceinline__ void mma32(f32x4& acc, s16x8 a, s16x8 b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                acc, 0, 0, 0);
}

__device__ __forceinline__ float lo_bf16(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// 4 floats -> 4 bf16 (RNE) stored as 8 bytes
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  return uint2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t seq_rsrc(const void* base, long first_elem, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(static_cast<const void*>(static_cast<const unsigned short*>(base) + first_elem)),
      (short)0, bytes, kBufferFlags);
}
// per-lane byte offset plus a wave-uniform one (kept in a scalar register)
__device__ __forceinline__ uint4 ld16s(__amdgpu_buffer_rsrc_t rs, unsigned voff, unsigned soff) {
  const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff, (int)soff, 0);
  return uint4{x[0], x[1], x[2], x[3]};
}
__device__ __forceinline__ uint2 ld8s(__amdgpu_buffer_rsrc_t rs, unsigned voff, unsigned soff) {
  const auto x = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)voff, (int)soff, 0);
  return uint2{x[0], x[1]};
}

// Hides a value from the optimiser, so that addresses derived from it are formed
// inside the chunk loop instead of being hoisted into dozens of live registers.
__device__ __forceinline__ void pipe_launder(unsigned& x) { asm volatile("" : "+v"(x)); }

// DPP shifts toward lower lanes inside a row of 16 (lane m reads m + k; past the
// row's end reads 0)
constexpr int kRowShl1 = 0x101, kRowShl2 = 0x102, kRowShl4 = 0x104, kRowShl8 = 0x108;

// Sequence geometry of a unit: its rows in the [.., T, d] tensors, its length,
// and the first workspace slot of its chunk states.
struct Seq {
  long r0;     // first row
  long len;    // tokens
  long slot0;  // workspace slot of chunk 0 (per head: n + start / 64)
};
__device__ __forceinline__ Seq seq_of(const BwdParams& prm, int n, int h) {
  Seq s;
  if (prm.cu) {
    const long bos = prm.cu[n], eos = prm.cu[n + 1];
    s.r0 = (long)h * prm.T + bos;
    s.len = eos - bos;
    s.slot0 = (long)h * prm.slots + n + bos / C;
  } else {
    s.r0 = ((long)n * prm.H + h) * prm.T;
    s.len = prm.T;
    s.slot0 = (long)h * prm.slots + n + (long)n * prm.T / C;
  }
  return s;
}

}  // namespace bwd

// ============================================================================
// Backward main kernel: one workgroup (8 waves) per (sequence, head).
//
// Wave w < DK/16 owns key channels [16w, 16w+16) of both carried states, all
// d_v columns, as H^T / B^T accumulator tiles: lane (m, grp) of tile nb holds
// columns 16nb + 4grp + 0..3 of channel 16w + m.  For a 32-column contraction
// step kk, tiles 2kk and 2kk+1 are then exactly a 16x16x32 operand (slots 0-3
// <-> columns 32kk + 4grp + r, slots 4-7 <-> 32kk + 16 + 4grp + r), so the
// inter terms of dq and dk read the state from registers; only dv, which
// contracts over channels, needs the bf16 state in LDS.  The same wave owns
// dq, dk and dg of its channels, so the gate-gradient boundary term and the
// in-chunk reverse sums stay inside the wave.  Wave w < DV/16 computes dv for
// columns [16w, 16w+16).
// ============================================================================
// SLICED: one column slice of a wider d_v (prm.pmode sums dq, dk and dg over the
// slices); otherwise they are written directly, with no per-store test.
template <int DK, int DV, bool SLICED>
__global__ __launch_bounds__(512, 1) void chunk_bwd_kernel(BwdParams prm) {
  using namespace bwd;
  constexpr unsigned RD = DK * 4;  // bytes per row of the fp32 Delta tile
  constexpr int LP = L + 8;        // [i][j] 16x16 score tile pitch (elements)
  constexpr int CB = DK / 16, NB = DV / 16;
  constexpr int NCG = DK / 8;
  constexpr int NGL = 16 * NCG;             // gating lanes per half (waves 0.. and 4..)
  constexpr int NVU = DV / 8;               // 16-byte units per value row
  constexpr int NCP = C * NVU / 512;        // units per lane of the value and dO copies
  static_assert(NGL <= 256 && NCP >= 1, "shape");

  // bf16 tiles with swizzled 256-byte rows (see swz), then the unswizzled rest
  struct Smem {
    char qs[C * 256];              // q~  [token][channel]
    char ks[C * 256];              // k~  [token][channel]
    char vs[C * 256];              // v   [token][column]
    char os[C * 256];              // dO  [token][column]
    char ss[DK * 256];             // B^ (bf16) [channel][column]
    char dl[C * RD];               // Delta = Gamma - b_s (log2), fp32 [token][channel], swizzled units
    unsigned short as[NS][L * LP]; // A = dO V^T of sub-chunk s, [i][j], j <= i
    unsigned short ps[NS][L * LP]; // P = q~ k~^T of sub-chunk s, [i][j], j <= i
    float fac[NS + 1][DK];         // state factors: 2^b_0, 2^(b_s - b_{s-1}) (s = 1..3), 2^(Gamma_last - b_3)
  };
  __shared__ __attribute__((aligned(256))) Smem sm;
  char* const lds = reinterpret_cast<char*>(&sm);
  constexpr unsigned oQ = offsetof(Smem, qs), oK = offsetof(Smem, ks), oV = offsetof(Smem, vs),
                     oO = offsetof(Smem, os), oS = offsetof(Smem, ss), oA = offsetof(Smem, as),
                     oP = offsetof(Smem, ps), oD = offsetof(Smem, dl), oF = offsetof(Smem, fac);
  static_assert(oQ % 256 == 0 && oK % 256 == 0 && oV % 256 == 0 && oO % 256 == 0 && oS % 256 == 0 &&
                oD % 256 == 0, "swizzled tiles start on 256-byte boundaries");
  auto rd8 = [&](unsigned off) __attribute__((always_inline)) {
    return *reinterpret_cast<const s16x4*>(lds + off);
  };
  auto rd16 = [&](unsigned off) __attribute__((always_inline)) {
    return *reinterpret_cast<const s16x8*>(lds + off);
  };
  auto rdt = [&](unsigned off) __attribute__((always_inline)) { return tr_read(reinterpret_cast<const unsigned short*>(lds + off)); };
  auto cat = [](s16x4 a, s16x4 b) __attribute__((always_inline)) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool sw = wave < CB;   // owns channels c0.. of the states, dq, dk, dg
  const bool vw = wave < NB;   // computes dv for columns n0..
  const int c0 = 16 * wave, n0 = 16 * wave;
  const int item = blockIdx.x;                 // (unit, segment)
  const int unit = item / prm.nseg, seg = item - unit * prm.nseg;
  const int n = unit / prm.H, h = unit - n * prm.H;
  const Seq sq = seq_of(prm, n, h);
  const int nch = (int)((sq.len + C - 1) / C);
  const int u_lo = seg * (prm.seg_len / C);  // chunks [u_lo, u_hi) of this work item
  const int u_hi = min(nch, (seg + 1) * (prm.seg_len / C));
  const __amdgpu_buffer_rsrc_t rs_q = seq_rsrc(prm.q, sq.r0 * DK, (int)(sq.len * DK * 2));
  const __amdgpu_buffer_rsrc_t rs_k = seq_rsrc(prm.k, sq.r0 * DK, (int)(sq.len * DK * 2));
  const __amdgpu_buffer_rsrc_t rs_g = seq_rsrc(prm.g, sq.r0 * DK, (int)(sq.len * DK * 2));
  // this launch's columns [col0, col0 + DV) of rows LDV long; reads past the
  // sequence's last row fall outside the record and return zeros
  // (one slice of width DV: prm.ldv == DV and prm.col0 == 0, known at compile time)
  const int LDV = SLICED ? prm.ldv : DV, col0 = SLICED ? prm.col0 : 0;
  const int v_bytes = sq.len > 0 ? (int)(sq.len * LDV * 2 - col0 * 2) : 0;
  const __amdgpu_buffer_rsrc_t rs_v = seq_rsrc(prm.v, sq.r0 * LDV + col0, v_bytes);
  const __amdgpu_buffer_rsrc_t rs_o = seq_rsrc(prm.dout, sq.r0 * LDV + col0, v_bytes);
  // this unit's chunk-start states (bf16 [chunk][dk][LDV])
  const __amdgpu_buffer_rsrc_t rs_h =
      seq_rsrc(prm.hs, sq.slot0 * DK * LDV, (int)((long)(nch > 0 ? nch : 1) * DK * LDV * 2));
  unsigned short* const dq_out = static_cast<unsigned short*>(prm.dq) + sq.r0 * DK;
  unsigned short* const dk_out = static_cast<unsigned short*>(prm.dk) + sq.r0 * DK;
  unsigned short* const dg_out = static_cast<unsigned short*>(prm.dg) + sq.r0 * DK;
  unsigned short* const dv_out = static_cast<unsigned short*>(prm.dv) + sq.r0 * LDV + col0;
  // dq, dk or dg (which = 0, 1, 2) at element e of this unit's [len][DK] rows: written
  // directly, or summed over the column slices in fp32 (prm.pmode)
  auto put = [&](unsigned short* out, int which, long e, float x0, float x1, float x2, float x3)
                 __attribute__((always_inline)) {
    if (!SLICED) {
      *reinterpret_cast<uint2*>(out + e) = pack4(x0, x1, x2, x3);
      return;
    }
    float4* const pp = reinterpret_cast<float4*>(prm.part + ((long)which * prm.part_rows + sq.r0) * DK + e);
    if (prm.pmode != 1) {
      const float4 y = *pp;
      x0 += y.x; x1 += y.y; x2 += y.z; x3 += y.w;
    }
    if (prm.pmode == 3)
      *reinterpret_cast<uint2*>(out + e) = pack4(x0, x1, x2, x3);
    else
      *pp = make_float4(x0, x1, x2, x3);
  };

  // ---- lane roles for the load phase ------------------------------------------
  // Both halves of the workgroup scan the gates, lane (tg, cg) of each half over
  // tokens 4tg..+3 and channels 8cg..+7, with the same code and so the same
  // values: the first half builds q~, the Delta tile and the state factors, the
  // second half k~.  Every lane copies a share of the values and dO.
  // Both are wave-uniform (NGL is a multiple of 64): the q/k loads of a wave then
  // keep one scalar buffer descriptor instead of a per-lane choice between two,
  // which the compiler would have to issue as a loop over the distinct values.
  const bool ql = wave < NGL / 64;                    // query-side gating wave
  const bool kl = wave >= 4 && wave < 4 + NGL / 64;   // key-side gating wave
  // Lane-dependent offsets are recomputed where they are used, from an opaque
  // copy of the lane index: kept live across the chunk loop they would not fit
  // beside the states, and their spill reloads would wait for every
  // outstanding global access.
  auto fresh_tid = [&]() __attribute__((always_inline)) {
    unsigned t = (unsigned)threadIdx.x;
    pipe_launder(t);
    return (int)t;
  };

  // Next chunk's raw inputs: q or k rows (pf[0..3]) and g rows (pf[4..7]) of a
  // gating lane, then the lane's v and dO units (pf[8..]).
  constexpr int NPF = 8 + 2 * NCP;
  uint4 pf[NPF];
  uint2 rh[NB];   // the chunk-start state of this wave's channels
  auto prefetch = [&](int u) __attribute__((always_inline)) {
    const int tl = fresh_tid();
    const int tg = tl & 15, cg = (tl & 255) >> 4;
    const unsigned qk_lane = (unsigned)((4 * tg) * DK + 8 * cg) * 2u;
    if (ql) {
#pragma unroll
      for (int a = 0; a < 4; ++a) pf[a] = ld16s(rs_q, qk_lane, (unsigned)(u * C + a) * DK * 2u);
    } else if (kl) {
#pragma unroll
      for (int a = 0; a < 4; ++a) pf[a] = ld16s(rs_k, qk_lane, (unsigned)(u * C + a) * DK * 2u);
    }
    if (ql || kl) {
#pragma unroll
      for (int a = 0; a < 4; ++a) pf[4 + a] = ld16s(rs_g, qk_lane, (unsigned)(u * C + a) * DK * 2u);
    }
#pragma unroll
    for (int it = 0; it < NCP; ++it) {
      const int idx = tl + 512 * it, row = idx / NVU, un = idx % NVU;
      const unsigned so = (unsigned)(u * C) * LDV * 2u;
      pf[8 + it] = ld16s(rs_v, (unsigned)(row * LDV + 8 * un) * 2u, so);
      pf[8 + NCP + it] = ld16s(rs_o, (unsigned)(row * LDV + 8 * un) * 2u, so);
    }
  };
  auto prefetch_state = [&](int u) __attribute__((always_inline)) {
    const int tl = fresh_tid();
    // channel c0 + m, columns 16 b + 4 grp .. + 3: 8 contiguous bytes of the slot
    const unsigned h_lane = 2u * (unsigned)chunk_state_index(c0 + (tl & 15), 4 * ((tl >> 4) & 3), DK);
    if (sw) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
        rh[b] = ld8s(rs_h, h_lane + 32u * DK * (unsigned)(b + col0 / 16), (unsigned)u * DK * LDV * 2u);
    }
  };

  // the state gradient entering this work item from later tokens: dS_T, or the
  // segment scan's result when the sequence is split
  f32x4 Ht[NB], Bt[NB];
  const float* const b_in = prm.nseg > 1 ? prm.seg_state + (long)item * DK * LDV
                                         : (prm.dsT ? prm.dsT + (long)unit * DK * LDV : nullptr);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    Bt[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (sw && b_in) {
      const float4 x = *reinterpret_cast<const float4*>(b_in + (long)(c0 + m) * LDV + col0 + 16 * b + 4 * grp);
      Bt[b] = f32x4{x.x, x.y, x.z, x.w};
    }
  }
  if (u_hi > u_lo) {
    prefetch(u_hi - 1);
    prefetch_state(u_hi - 1);
  }

  // bf16 operand of a 32-column step from two state tiles (see the kernel comment)
  auto state_op = [](const f32x4& a, const f32x4& b) __attribute__((always_inline)) {
    return __builtin_bit_cast(s16x8, uint4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                           pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])});
  };

  for (int u = u_hi - 1; u >= u_lo; --u) {
    const long row0 = (long)u * C;   // first token of this chunk (sequence-relative)
    // ======================= load phase =======================
    if (ql || kl) {
      const int tl = fresh_tid();
      const int tg = tl & 15, cg = (tl & 255) >> 4;
      // log2 cumulative gate over the chunk, per channel
      float gm[4][8];
      const unsigned* gw[4] = {&pf[4].x, &pf[5].x, &pf[6].x, &pf[7].x};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const unsigned w = gw[a][i >> 1];
          const float y = ((i & 1) ? hi_bf16(w) : lo_bf16(w)) * kLog2e;
          gm[a][i] = a ? gm[a - 1][i] + y : y;
        }
        float x = gm[3][i];
        x += dpp<kRowShr1>(x);
        x += dpp<kRowShr2>(x);
        x += dpp<kRowShr4>(x);
        x += dpp<kRowShr8>(x);
        const float ex = x - gm[3][i];
#pragma unroll
        for (int a = 0; a < 4; ++a) gm[a][i] += ex;
      }
      const int s = tg >> 2;   // this lane's sub-chunk
      const unsigned* xw[4] = {&pf[0].x, &pf[1].x, &pf[2].x, &pf[3].x};   // q or k rows
      // The carried states move between sub-chunks by one factor each:
      // 2^(Gamma_{s-1,last} - b_{s-1}) 2^(b_s - Gamma_{s-1,last}) = 2^(b_s - b_{s-1}).
      float piv[8], f0[8], f1[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float first = quad_bcast_c<0>(gm[0][i]);   // Gamma at the sub-chunk's first row
        const float last = quad_bcast_c<3>(gm[3][i]);    // ... and at its last row
        float b = 0.5f * (first + last);
        if (!(first - last <= kRangeLimit)) b = __int_as_float(0x7fc00000);
        piv[i] = b;
        f0[i] = fast_exp2(b - dpp<kRowShr4>(b));          // previous sub-chunk's pivot (0 for s = 0)
        f1[i] = fast_exp2(last - b);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float xv[8], dv8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float d = gm[a][i] - piv[i];
          dv8[i] = d;
          const unsigned wx = xw[a][i >> 1];
          xv[i] = ((i & 1) ? hi_bf16(wx) : lo_bf16(wx)) * fast_exp2(ql ? d : -d);   // q~ or k~
        }
        // row 4 tg + a: unit cg of the token tiles, units 2 cg and 2 cg + 1 of Delta
        const unsigned wt = (toff(4 * tg, cg, 0) ^ cx(a, 0)) + ca(a, 0);
        *reinterpret_cast<uint4*>(lds + (ql ? oQ : oK) + wt) =
            uint4{pack_bf16x2(xv[0], xv[1]), pack_bf16x2(xv[2], xv[3]), pack_bf16x2(xv[4], xv[5]),
                  pack_bf16x2(xv[6], xv[7])};
        if (ql) {
          const unsigned wd = toff(4 * tg, 2 * cg, 0, RD);
          *reinterpret_cast<float4*>(lds + oD + ((wd ^ cx(a, 0)) + ca(a, 0, RD))) =
              make_float4(dv8[0], dv8[1], dv8[2], dv8[3]);
          *reinterpret_cast<float4*>(lds + oD + ((wd ^ cx(a, 1)) + ca(a, 1, RD))) =
              make_float4(dv8[4], dv8[5], dv8[6], dv8[7]);
        }
      }
      if (ql && (tg & 3) == 0) {
        *reinterpret_cast<float4*>(&sm.fac[s][8 * cg]) = make_float4(f0[0], f0[1], f0[2], f0[3]);
        *reinterpret_cast<float4*>(&sm.fac[s][8 * cg + 4]) = make_float4(f0[4], f0[5], f0[6], f0[7]);
        if (s == NS - 1) {
          *reinterpret_cast<float4*>(&sm.fac[NS][8 * cg]) = make_float4(f1[0], f1[1], f1[2], f1[3]);
          *reinterpret_cast<float4*>(&sm.fac[NS][8 * cg + 4]) = make_float4(f1[4], f1[5], f1[6], f1[7]);
        }
      }
    }
    {
      const int cp = fresh_tid();
#pragma unroll
      for (int it = 0; it < NCP; ++it) {   // row cp / NVU + it * 512 / NVU, unit cp % NVU
        constexpr unsigned RI = 512 / NVU;
        const unsigned wc = (toff(cp / NVU, cp % NVU, 0) ^ cx(RI * it, 0)) + ca(RI * it, 0);
        *reinterpret_cast<uint4*>(lds + oV + wc) = pf[8 + it];
        *reinterpret_cast<uint4*>(lds + oO + wc) = pf[8 + NCP + it];
      }
    }
    barrier_lds();
    // Per-lane LDS byte offsets (wave parts included); every access adds a
    // compile-time constant, which the DS instructions take as an immediate.
    // Computed after the load phase, from an opaque lane index, so that they
    // are neither live during it nor kept across the loop.
    const int tl = fresh_tid();
    const int m = tl & 15, grp = (tl >> 4) & 3;
    // swizzled tiles (row, unit, byte; see toff):
    unsigned r16 = toff(m, grp >> 1, 8 * (grp & 1));                 // 8 B at column 4 grp of row m
    unsigned r32 = toff(m, grp, 0);                                  // 16 B at column 8 grp of row m
    unsigned tV = toff(4 * grp + (m >> 2), (m & 3) >> 1, 8 * (m & 1));   // transposing: rows 4grp + m/4
    unsigned tW = toff(4 * grp + (m >> 2), 2 * wave + ((m & 3) >> 1), 8 * (m & 1));   // ... at column 16 wave
    unsigned tS = toff(8 * grp + (m >> 2), 2 * wave + ((m & 3) >> 1), 8 * (m & 1));   // state rows 8grp + m/4
    unsigned wS = toff(c0 + m, grp >> 1, 8 * (grp & 1));             // state tile writes, row c0 + m
    unsigned eQ = toff(m, 2 * wave + (grp >> 1), 8 * (grp & 1));     // channels c0 + 4 grp of row m
    unsigned eD = toff(m, 4 * wave + grp, 0, RD);                    // the same in the Delta tile
    // 16x16 score tiles (row pitch LP)
    unsigned tL = ((4 * grp + (m >> 2)) * LP + 4 * (m & 3)) * 2;     // transposed
    unsigned r16L = (m * LP + 4 * grp) * 2;
    unsigned fC = (c0 + m) * 4;
    pipe_launder(r16); pipe_launder(r32); pipe_launder(tV); pipe_launder(tW); pipe_launder(tS);
    pipe_launder(wS); pipe_launder(eQ); pipe_launder(eD); pipe_launder(tL); pipe_launder(r16L);
    pipe_launder(fC);
    // address of a swizzled-tile access: lane part ln, compile-time row r and unit u
    auto at = [](unsigned ln, unsigned r, unsigned u) __attribute__((always_inline)) {
      return (ln ^ cx(r, u)) + ca(r, u);
    };


    // =============== score blocks of the four sub-chunks ===============
    {
      const int s = wave & 3;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const unsigned b = toff(16 * s + m, grp, 0);   // 16 B at column 8 grp of row 16 s + m
      if (wave < 4) {   // A^T[j][i] = sum_n v_j[n] dO_i[n]
#pragma unroll
        for (int kk = 0; kk < DV / 32; ++kk) mma32(acc, rd16(oV + at(b, 0, 4 * kk)), rd16(oO + at(b, 0, 4 * kk)));
      } else {          // P^T[j][i] = sum_c k~_j[c] q~_i[c]
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) mma32(acc, rd16(oK + at(b, 0, 4 * kk)), rd16(oQ + at(b, 0, 4 * kk)));
      }
      // lane holds rows j = 4 grp + r at column i = m; keep j <= i, store as [i][j]
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = (4 * grp + r <= m) ? acc[r] : 0.f;
      *reinterpret_cast<uint2*>(lds + (wave < 4 ? oA : oP) + s * L * LP * 2 + r16L) = pack4(x[0], x[1], x[2], x[3]);
    }
    barrier_lds();

    // ======================= forward sweep: dq =======================
    // the chunk-start state, widened only now (during the load phase its bf16
    // form takes half the registers) and scaled into H^ of sub-chunk 0
    if (sw) {
      const float f = *reinterpret_cast<const float*>(lds + oF + fC);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        Ht[b] = f32x4{lo_bf16(rh[b].x), hi_bf16(rh[b].x), lo_bf16(rh[b].y), hi_bf16(rh[b].y)} * f;
    }
    float qd[NS][4];   // q~ * (dq before its 2^Delta factor), for dg
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      // the next chunk's inputs are requested at the second sub-chunk: early enough
      // to arrive, and before most of this sweep's dq stores.  (Loads and stores
      // share vmcnt and may complete out of order, so a load whose registers
      // earlier stores read waits for every outstanding store.)
      if (s == 1 && u > u_lo) prefetch(u - 1);
      if (sw) {   // Ht holds H^ of sub-chunk s
        // k~^T[c][j] A[i][j] over j in the sub-chunk first: it does not wait for
        // the carried state, which the products after it do
        const s16x4 kt = rdt(oK + at(tW, 16 * s, 0));
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        mma16_add(acc, kt, rd8(oA + s * L * LP * 2 + r16L));
#pragma unroll
        for (int kk = 0; kk < DV / 32; ++kk)   // H^[c][n] dO[i][n]
          mma32(acc, state_op(Ht[2 * kk], Ht[2 * kk + 1]),
                cat(rd8(oO + at(r16, 16 * s, 4 * kk)), rd8(oO + at(r16, 16 * s, 4 * kk + 2))));
        // lane: channels c0 + 4 grp + r at token 16 s + m
        const float4 d = *reinterpret_cast<const float4*>(lds + oD + ((eD ^ cx(16 * s, 0)) + ca(16 * s, 0, RD)));
        const uint2 qv = *reinterpret_cast<const uint2*>(lds + oQ + at(eQ, 16 * s, 0));
        qd[s][0] = lo_bf16(qv.x) * acc[0];
        qd[s][1] = hi_bf16(qv.x) * acc[1];
        qd[s][2] = lo_bf16(qv.y) * acc[2];
        qd[s][3] = hi_bf16(qv.y) * acc[3];
        const long t = row0 + 16 * s + m;
        if (t < sq.len)
          put(dq_out, 0, t * DK + c0 + 4 * grp, fast_exp2(d.x) * acc[0], fast_exp2(d.y) * acc[1],
              fast_exp2(d.z) * acc[2], fast_exp2(d.w) * acc[3]);
        // H^ + k~^T V over the sub-chunk's tokens, then the factor to H^ of
        // sub-chunk s + 1 (after the last one: to H at the chunk's end)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          mma16(Ht[b], rdt(oV + at(tV, 16 * s, 2 * b)), kt);
        const float f = *reinterpret_cast<const float*>(lds + oF + (s + 1) * DK * 4 + fC);
#pragma unroll
        for (int b = 0; b < NB; ++b) Ht[b] = Ht[b] * f;
      }
    }

    // ===== gate gradient at the chunk end: sum_n H[c][n] B[c][n] per channel =====
    float carry[4] = {0.f, 0.f, 0.f, 0.f};
    if (sw) {
      float p = 0.f;
#pragma unroll
      for (int b = 0; b < NB; ++b)
        p += Ht[b][0] * Bt[b][0] + Ht[b][1] * Bt[b][1] + Ht[b][2] * Bt[b][2] + Ht[b][3] * Bt[b][3];
      p += __shfl_xor(p, 16);
      p += __shfl_xor(p, 32);   // channel c0 + m, in every lane of column m
#pragma unroll
      for (int r = 0; r < 4; ++r) carry[r] = __shfl(p, 4 * grp + r);
    }
    // H is not needed again in this chunk: its registers take the next chunk's state
    if (u > u_lo) prefetch_state(u - 1);

    // ======================= reverse sweep: dk, dv, dg =======================
    if (sw) {   // B^ of sub-chunk 3 = 2^(Gamma_last - b_3) B
      const float f = *reinterpret_cast<const float*>(lds + oF + NS * DK * 4 + fC);
#pragma unroll
      for (int b = 0; b < NB; ++b) Bt[b] = Bt[b] * f;
    }
#pragma unroll
    for (int s = NS - 1; s >= 0; --s) {
      if (sw) {   // Bt holds B^ of sub-chunk s; its bf16 copy for dv
#pragma unroll
        for (int b = 0; b < NB; ++b)
          *reinterpret_cast<uint2*>(lds + oS + at(wS, 0, 2 * b)) = pack4(Bt[b][0], Bt[b][1], Bt[b][2], Bt[b][3]);
      }
      barrier_lds();
      if (sw) {
        // q~^T[c][i] A[i][j] over i in the sub-chunk first (independent of B^)
        const s16x4 qt = rdt(oQ + at(tW, 16 * s, 0));
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        mma16_add(acc, qt, rdt(oA + s * L * LP * 2 + tL));
#pragma unroll
        for (int kk = 0; kk < DV / 32; ++kk)   // B^[c][n] v[j][n]
          mma32(acc, state_op(Bt[2 * kk], Bt[2 * kk + 1]),
                cat(rd8(oV + at(r16, 16 * s, 4 * kk)), rd8(oV + at(r16, 16 * s, 4 * kk + 2))));
        const float4 d = *reinterpret_cast<const float4*>(lds + oD + ((eD ^ cx(16 * s, 0)) + ca(16 * s, 0, RD)));
        const uint2 kv = *reinterpret_cast<const uint2*>(lds + oK + at(eQ, 16 * s, 0));
        float x[4] = {qd[s][0] - lo_bf16(kv.x) * acc[0], qd[s][1] - hi_bf16(kv.x) * acc[1],
                      qd[s][2] - lo_bf16(kv.y) * acc[2], qd[s][3] - hi_bf16(kv.y) * acc[3]};
        // reverse inclusive sum over the 16 tokens of the sub-chunk (lanes m)
        float dgv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float y = x[r];
          y += dpp<kRowShl1>(y);
          y += dpp<kRowShl2>(y);
          y += dpp<kRowShl4>(y);
          y += dpp<kRowShl8>(y);
          dgv[r] = y + carry[r];
          carry[r] += __shfl(y, lane & 48);
        }
        const long t = row0 + 16 * s + m;
        if (t < sq.len) {
          put(dk_out, 1, t * DK + c0 + 4 * grp, fast_exp2(-d.x) * acc[0], fast_exp2(-d.y) * acc[1],
              fast_exp2(-d.z) * acc[2], fast_exp2(-d.w) * acc[3]);
          put(dg_out, 2, t * DK + c0 + 4 * grp, dgv[0], dgv[1], dgv[2], dgv[3]);
        }
        // B^ + q~^T dO over the sub-chunk's tokens, then the factor to B^ of
        // sub-chunk s - 1 (after the first one: to B at the chunk's start)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          mma16(Bt[b], rdt(oO + at(tV, 16 * s, 2 * b)), qt);
        const float f = *reinterpret_cast<const float*>(lds + oF + s * DK * 4 + fC);
#pragma unroll
        for (int b = 0; b < NB; ++b) Bt[b] = Bt[b] * f;
      }
      if (vw) {
        // dO^T[n][i] P[i][j] over i in the sub-chunk, then B^^T[n][c] k~[j][c]
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        mma16_add(acc, rdt(oO + at(tW, 16 * s, 0)), rdt(oP + s * L * LP * 2 + tL));
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk)
          mma32(acc, cat(rdt(oS + at(tS, 32 * kk, 0)), rdt(oS + at(tS, 32 * kk + 4, 0))),
                rd16(oK + at(r32, 16 * s, 4 * kk)));
        const long t = row0 + 16 * s + m;
        if (t < sq.len)
          *reinterpret_cast<uint2*>(dv_out + t * LDV + n0 + 4 * grp) = pack4(acc[0], acc[1], acc[2], acc[3]);
      }
      barrier_lds();
    }
  }

  if (sw && prm.ds0 && seg == 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      *reinterpret_cast<float4*>(prm.ds0 + ((long)unit * DK + c0 + m) * LDV + col0 + 16 * b + 4 * grp) =
          make_float4(Bt[b][0], Bt[b][1], Bt[b][2], Bt[b][3]);
  }
}

int launch_chunk_bwd(const BwdParams& prm, int dk, int dv, int nblocks, hipStream_t stream) {
#define GLA_BWD(K, V)                                                                          \
  do {                                                                                         \
    if (prm.pmode)                                                                             \
      hipLaunchKernelGGL((chunk_bwd_kernel<K, V, true>), dim3(nblocks), dim3(512), 0, stream, prm);  \
    else                                                                                       \
      hipLaunchKernelGGL((chunk_bwd_kernel<K, V, false>), dim3(nblocks), dim3(512), 0, stream, prm); \
  } while (0)
  if (dk == 128 && dv == 128)
    GLA_BWD(128, 128);
  else if (dk == 128 && dv == 64)
    GLA_BWD(128, 64);
  else if (dk == 64 && dv == 128)
    GLA_BWD(64, 128);
  else if (dk == 64 && dv == 64)
    GLA_BWD(64, 64);
  else
    return -2;
#undef GLA_BWD
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gla
