// C ABI of libgla.so (declared in include/gla.h): argument validation on the
// host, kernel selection and launch.  Nothing here computes: every step of the
// forward pass and of the decode step runs in the HIP kernels.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "gla.h"
#include "gla_kernels.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool fits_i32(long long x) { return x >= 0 && x <= 0x7fffffffLL; }

}  // namespace

extern "C" {

const char* gla_status_string(int status) {
  switch (status) {
    case GLA_OK: return "GLA_OK";
    case GLA_ERR_INVALID_ARG: return "GLA_ERR_INVALID_ARG";
    case GLA_ERR_UNSUPPORTED: return "GLA_ERR_UNSUPPORTED";
    case GLA_ERR_LAUNCH: return "GLA_ERR_LAUNCH";
    default: return "GLA_UNKNOWN_STATUS";
  }
}

const char* gla_last_error(void) { return g_last_error; }

int gla_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                  const float* initial_state, void* o, float* final_state,
                  const int32_t* cu_seqlens, int num_seqs, int B, int H, int T, int dk,
                  int dv, int chunk_size, int dtype, void* stream) {
  g_last_error[0] = '\0';
  if (dtype != GLA_BF16 && dtype != GLA_F32)
    return fail(GLA_ERR_INVALID_ARG, "gla_chunk_fwd: dtype %d is not GLA_BF16 or GLA_F32", dtype);
  if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0)
    return fail(GLA_ERR_INVALID_ARG, "gla_chunk_fwd: B=%d H=%d T=%d dk=%d dv=%d must be positive (T >= 0)",
                B, H, T, dk, dv);
  if (chunk_size != 64)
    return fail(GLA_ERR_UNSUPPORTED, "gla_chunk_fwd: chunk_size %d (only 64 is implemented)", chunk_size);
  if (dtype == GLA_BF16 ? (dk != 64 && dk != 128) : dk != 64)
    return fail(GLA_ERR_UNSUPPORTED, "gla_chunk_fwd: dk=%d is not implemented for %s", dk,
                dtype == GLA_BF16 ? "GLA_BF16 (64 or 128)" : "GLA_F32 (64)");
  if (dv % 64 != 0 || dv > 512)
    return fail(GLA_ERR_UNSUPPORTED, "gla_chunk_fwd: dv=%d must be a multiple of 64 up to 512", dv);
  int nseq = B;
  if (cu_seqlens) {
    if (B != 1)
      return fail(GLA_ERR_INVALID_ARG, "gla_chunk_fwd: packed sequences (cu_seqlens) need B == 1, got %d", B);
    if (num_seqs <= 0)
      return fail(GLA_ERR_INVALID_ARG, "gla_chunk_fwd: num_seqs=%d must be positive with cu_seqlens",
                  num_seqs);
    nseq = num_seqs;
  }
  if (!fits_i32((long long)B * H * T) || !fits_i32((long long)B * H * T * dv) ||
      !fits_i32((long long)B * H * T * dk) || !fits_i32((long long)nseq * H * dk * dv))
    return fail(GLA_ERR_INVALID_ARG, "gla_chunk_fwd: tensor sizes exceed int32 indexing");
  const bool any_tokens = (long long)B * H * T > 0;
  if (any_tokens && (!q || !k || !v || !g || !o))
    return fail(GLA_ERR_INVALID_ARG, "gla_chunk_fwd: q, k, v, g and o must be non-null");
  const void* ptrs[] = {q, k, v, g, o, initial_state, final_state, cu_seqlens};
  const char* names[] = {"q", "k", "v", "g", "o", "initial_state", "final_state", "cu_seqlens"};
  for (int i = 0; i < 8; ++i)
    if (ptrs[i] && !aligned16(ptrs[i]))
      return fail(GLA_ERR_INVALID_ARG, "gla_chunk_fwd: %s is not 16-byte aligned", names[i]);
  const long long units = (long long)nseq * H;
  const int nvt = dv / 64;
  const long long nblocks = units * nvt;
  if (!fits_i32(nblocks) || nblocks == 0)
    return fail(GLA_ERR_INVALID_ARG, "gla_chunk_fwd: %lld work items", nblocks);
  if (!any_tokens && !final_state) return GLA_OK;  // nothing to compute or write

  gla::ChunkParams prm;
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.g = g;
  prm.s0 = initial_state;
  prm.o = o;
  prm.sT = final_state;
  prm.cu = cu_seqlens;
  prm.H = H;
  prm.T = T;
  prm.DV = dv;
  prm.nvt = nvt;
  prm.xcd_remap = (nblocks % 8 == 0) ? 1 : 0;
  const int rc = gla::launch_chunk_fwd(prm, dk, dtype, (int)nblocks,
                                       reinterpret_cast<hipStream_t>(stream));
  if (rc == -2) return fail(GLA_ERR_UNSUPPORTED, "gla_chunk_fwd: no kernel for dk=%d dtype=%d", dk, dtype);
  if (rc != 0)
    return fail(GLA_ERR_LAUNCH, "gla_chunk_fwd: kernel launch failed: %s",
                hipGetErrorString(hipGetLastError()));
  return GLA_OK;
}

int gla_recurrent_step(const void* q, const void* k, const void* v, const void* g, float* state,
                       void* o, int N, int H, int dk, int dv, int dtype, void* stream) {
  g_last_error[0] = '\0';
  if (dtype != GLA_BF16 && dtype != GLA_F32)
    return fail(GLA_ERR_INVALID_ARG, "gla_recurrent_step: dtype %d is not GLA_BF16 or GLA_F32", dtype);
  if (N <= 0 || H <= 0 || dk <= 0 || dv <= 0)
    return fail(GLA_ERR_INVALID_ARG, "gla_recurrent_step: N=%d H=%d dk=%d dv=%d must be positive", N, H,
                dk, dv);
  if ((dk != 64 && dk != 128 && dk != 256) || (dv != 64 && dv != 128 && dv != 256))
    return fail(GLA_ERR_UNSUPPORTED, "gla_recurrent_step: dk=%d dv=%d (each must be 64, 128 or 256)", dk,
                dv);
  if (!fits_i32((long long)N * H) || !fits_i32((long long)N * H * dk * dv))
    return fail(GLA_ERR_INVALID_ARG, "gla_recurrent_step: tensor sizes exceed int32 indexing");
  if (!q || !k || !v || !g || !state || !o)
    return fail(GLA_ERR_INVALID_ARG, "gla_recurrent_step: q, k, v, g, state and o must be non-null");
  const void* ptrs[] = {q, k, v, g, state, o};
  const char* names[] = {"q", "k", "v", "g", "state", "o"};
  for (int i = 0; i < 6; ++i)
    if (!aligned16(ptrs[i]))
      return fail(GLA_ERR_INVALID_ARG, "gla_recurrent_step: %s is not 16-byte aligned", names[i]);
  gla::StepParams prm;
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.g = g;
  prm.state = state;
  prm.o = o;
  const int rc = gla::launch_recurrent_step(prm, N * H, dk, dv, dtype,
                                            reinterpret_cast<hipStream_t>(stream));
  if (rc == -2)
    return fail(GLA_ERR_UNSUPPORTED, "gla_recurrent_step: no kernel for dk=%d dv=%d dtype=%d", dk, dv,
                dtype);
  if (rc != 0)
    return fail(GLA_ERR_LAUNCH, "gla_recurrent_step: kernel launch failed: %s",
                hipGetErrorString(hipGetLastError()));
  return GLA_OK;
}

}  // extern "C"
