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
  int nvt;           // DV / 64 column slices
  int xcd_remap;     // 1: consecutive work items share an XCD (grid size % 8 == 0)
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

// Each returns 0 on success, -1 if the launch failed, -2 if no kernel exists
// for the shape/dtype.
int launch_chunk_fwd(const ChunkParams& prm, int dk, int dtype, int nblocks, hipStream_t stream);
int launch_chunk_fwd_pipe(const ChunkParams& prm, int dk, int nblocks, hipStream_t stream);
int launch_recurrent_step(const StepParams& prm, int units, int dk, int dv, int dtype,
                          hipStream_t stream);

}  // namespace gla
