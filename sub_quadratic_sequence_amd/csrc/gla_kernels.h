// Internal launch interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace gla {

// Arguments of the chunkwise forward kernel (see include/gla.h for meanings).
struct ChunkParams {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const float* s0;   // may be null (zeros)
  void* o;
  float* sT;         // may be null (not written)
  const int* cu;     // packed varlen offsets on the device, or null
  int H;
  int T;             // tokens per sequence (fixed) or total packed tokens
  int DV;
  int dvt;           // columns per d_v slice: 64, or 128 (bf16 full pass only)
  int nvt;           // DV / dvt column slices
  int xcd_remap;     // 1: consecutive work items share an XCD (grid size % 8 == 0)
  // Sequence split (fixed-length inputs only; nseg = 1 and seg_len = T otherwise):
  // each sequence is cut into nseg segments of seg_len tokens (a multiple of 64,
  // the last one shorter), and a work item is one (sequence, head, segment, slice).
  int nseg;
  int seg_len;
  // Packed sequences: their count, and whether work items go longest sequence
  // first (nseq <= kMaxSortSeqs, nseq * H a multiple of 8, bf16 kernel).
  int nseq;
  int sort_units;
  float* seg_state;  // [units][nseg][dk][dv] fp32: a segment's state from zero, then its incoming state
  float* seg_decay;  // [units][nseg][dk] fp32: exp of the segment's summed log-gates
  // Chunk-state mode (the backward's recomputation): the state entering every
  // chunk, bf16, one dk x dv slot per chunk in the order of chunk_state_index.
  unsigned short* hs;
  int slots;         // slots per head: sequences + tokens / 64 + 1
};

constexpr int kMaxSortSeqs = 64;

// Kernel modes of the pipelined forward.
constexpr int kFull = 0;       // outputs (and the final state of unsplit sequences)
constexpr int kStateOnly = 1;  // a segment's state from zero and its total decay
constexpr int kChunkStates = 2;  // the state entering every chunk, to ChunkParams::hs
constexpr int kSegGrad = 3;      // the backward split's segment state gradients (k, v = q, dO)
constexpr int kFullStates = 4;   // kFull plus the state entering every chunk, to ChunkParams::hs

// Element (row c, column n) of a chunk-state slot (dk x dv, bf16): 16-column tiles
// of dk rows, each in blocks of 4 rows x 16 columns, a block as 4 groups of 4
// columns x the 4 rows x 4 columns.  A forward consumer lane stores 4 columns of
// one row (8 bytes) and each 16 lanes of a store instruction fill 128 contiguous
// bytes; a backward lane reads 4 columns of one row, and the four lanes of a quad
// (4 consecutive rows) read 32 contiguous bytes.
__host__ __device__ constexpr int chunk_state_index(int c, int n, int dk) {
  return (n >> 4) * (16 * dk) + (c >> 2) * 64 + ((n >> 2) & 3) * 16 + (c & 3) * 4 + (n & 3);
}

// Arguments of the segment scan of the sequence split.
struct SegScanParams {
  const float* s0;   // [units][dk][dv] or null (zeros)
  float* sT;         // [units][dk][dv] or null; may alias s0
  float* seg_state;  // in: states from zero; out: incoming states
  const float* seg_decay;
  int dk, dv, nseg;
  int reverse;       // 1: segments from last to first (the state gradient of the backward pass)
};

// Arguments of the decode step kernel.
struct StepParams {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  float* state;
  void* o;
};

// Arguments of the backward kernels (see include/gla.h for meanings).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* dout;      // gradient of the outputs
  const float* s0;       // initial state, or null (zeros)
  const float* dsT;      // gradient of the final state, or null (zeros)
  void* dq;
  void* dk;
  void* dv;
  void* dg;
  float* ds0;            // gradient of the initial state, or null (not written)
  unsigned short* hs;    // workspace: bf16 chunk-start states [H][slots][dk][dv]
  const int* cu;         // packed varlen offsets on the device, or null
  int H;
  int T;                 // tokens per sequence (fixed) or total packed tokens
  int DV;
  int nvt;               // DV / 64 column slices (state pass work items per unit)
  int slots;             // chunk-state slots per head: sequences + tokens / 64 + 1
  int xcd_remap;         // state pass: consecutive work items share an XCD
  // Sequence split (fixed-length inputs; nseg = 1 otherwise): nseg segments of
  // seg_len tokens (a multiple of 64, the last one shorter).  The backward work
  // items are (sequence, head, segment); a segment's incoming state gradient
  // comes from the gradient-state pass and the reverse segment scan.
  int nseg;
  int seg_len;
  float* seg_state;      // [units][nseg][dk][dv] fp32: a segment's state gradient from zero, then its incoming one
  float* seg_decay;      // [units][nseg][dk] fp32: exp of the segment's summed log-gates
  // Column slice of d_v handled by one backward launch (d_v above 128 runs as
  // slices of 128 or 64 columns in turn): ldv is the full d_v, the row stride of v,
  // d_o and d_v and the column count of every state-shaped tensor; col0 is the
  // slice's first column.
  int ldv;
  int col0;
  // dq, dk and dg summed over the slices: 0 one slice (bf16 written directly);
  // 1 the first slice (fp32 sums to part); 2 a middle slice (adds to part); 3 the
  // last slice (adds part's sums and writes bf16).
  int pmode;
  float* part;           // [3][part_rows][dk] fp32 partial dq, dk, dg (pmode != 0)
  long part_rows;        // rows of each partial tensor: B*H*T (packed: H*T)
};

// Arguments of the Gated DeltaNet chunk forward (see include/gla.h for meanings).
struct GdnParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g;      // [B, H, T] log forget gate
  const float* beta;   // [B, H, T] update gate
  const float* s0;     // may be null (zeros)
  void* o;
  float* sT;           // may be null (not written)
  const int* cu;       // packed varlen offsets on the device, or null
  int H;
  int T;               // tokens per sequence (fixed) or total packed tokens
  int DV;
  int nvt;             // DV / 64 column slices
  int xcd_remap;       // 1: consecutive work items share an XCD (grid size % 8 == 0)
};

// Each returns 0 on success, -1 if the launch failed, -2 if no kernel exists
// for the shape/dtype.
int launch_chunk_fwd(const ChunkParams& prm, int dk, int dtype, int nblocks, hipStream_t stream);
int launch_chunk_fwd_full_states(const ChunkParams& prm, int dk, int nblocks, hipStream_t stream);
int launch_chunk_fwd_pipe(const ChunkParams& prm, int dk, bool state_only, int nblocks,
                          hipStream_t stream);
int launch_chunk_fwd_states(const ChunkParams& prm, int dk, int nblocks, hipStream_t stream);
int launch_chunk_seg_grad(const ChunkParams& prm, int dk, int nblocks, hipStream_t stream);
int launch_seg_scan(const SegScanParams& prm, int units, hipStream_t stream);
int launch_chunk_bwd(const BwdParams& prm, int dk, int dv, int nblocks, hipStream_t stream);
int launch_gdn_chunk_fwd(const GdnParams& prm, int dk, int nblocks, hipStream_t stream);
int launch_recurrent_step(const StepParams& prm, int units, int dk, int dv, int dtype,
                          hipStream_t stream);

}  // namespace gla
