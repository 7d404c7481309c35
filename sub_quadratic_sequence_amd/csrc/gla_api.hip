// C ABI of libgla.so (declared in include/gla.h): argument validation on the
// host, kernel selection and launch.  Nothing here computes: every step of the
// forward pass and of the decode step runs in the HIP kernels.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "gla.h"
#include "gla_kernels.h"
#include "split_model.h"

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

}  // extern "C"

namespace {

// Host-side validation shared by the forward entry points; fills prm (unsplit)
// and the launch shape.  Returns GLA_OK, or an error status with the message set.
int check_chunk_args(const char* fn, const void* q, const void* k, const void* v, const void* g,
                     const float* initial_state, void* o, float* final_state,
                     const int32_t* cu_seqlens, int num_seqs, int B, int H, int T, int dk, int dv,
                     int chunk_size, int dtype, gla::ChunkParams& prm, long long& units,
                     bool& nothing_to_do) {
  nothing_to_do = false;
  if (dtype != GLA_BF16 && dtype != GLA_F32)
    return fail(GLA_ERR_INVALID_ARG, "%s: dtype %d is not GLA_BF16 or GLA_F32", fn, dtype);
  if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0)
    return fail(GLA_ERR_INVALID_ARG, "%s: B=%d H=%d T=%d dk=%d dv=%d must be positive (T >= 0)", fn,
                B, H, T, dk, dv);
  if (chunk_size != 64)
    return fail(GLA_ERR_UNSUPPORTED, "%s: chunk_size %d (only 64 is implemented)", fn, chunk_size);
  if (dk != 64 && dk != 128)
    return fail(GLA_ERR_UNSUPPORTED, "%s: dk=%d is not implemented (64 or 128)", fn, dk);
  if (dv % 64 != 0 || dv > 512)
    return fail(GLA_ERR_UNSUPPORTED, "%s: dv=%d must be a multiple of 64 up to 512", fn, dv);
  int nseq = B;
  if (cu_seqlens) {
    if (B != 1)
      return fail(GLA_ERR_INVALID_ARG, "%s: packed sequences (cu_seqlens) need B == 1, got %d", fn, B);
    if (num_seqs <= 0)
      return fail(GLA_ERR_INVALID_ARG, "%s: num_seqs=%d must be positive with cu_seqlens", fn,
                  num_seqs);
    nseq = num_seqs;
  }
  if (!fits_i32((long long)B * H * T) || !fits_i32((long long)B * H * T * dv) ||
      !fits_i32((long long)B * H * T * dk) || !fits_i32((long long)nseq * H * dk * dv))
    return fail(GLA_ERR_INVALID_ARG, "%s: tensor sizes exceed int32 indexing", fn);
  const bool any_tokens = (long long)B * H * T > 0;
  if (any_tokens && (!q || !k || !v || !g || !o))
    return fail(GLA_ERR_INVALID_ARG, "%s: q, k, v, g and o must be non-null", fn);
  const void* ptrs[] = {q, k, v, g, o, initial_state, final_state, cu_seqlens};
  const char* names[] = {"q", "k", "v", "g", "o", "initial_state", "final_state", "cu_seqlens"};
  for (int i = 0; i < 8; ++i)
    if (ptrs[i] && !aligned16(ptrs[i]))
      return fail(GLA_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, names[i]);
  units = (long long)nseq * H;
  const int nvt = dv / 64;
  const long long nblocks = units * nvt;
  if (!fits_i32(nblocks) || nblocks == 0)
    return fail(GLA_ERR_INVALID_ARG, "%s: %lld work items", fn, nblocks);
  if (!any_tokens && !final_state) nothing_to_do = true;

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
  prm.dvt = 64;
  prm.nvt = nvt;
  prm.xcd_remap = (nblocks % 8 == 0) ? 1 : 0;
  prm.nseg = 1;
  prm.seg_len = T;
  prm.seg_state = nullptr;
  prm.seg_decay = nullptr;
  prm.nseq = nseq;
  prm.sort_units = (cu_seqlens && dtype == GLA_BF16 && nseq <= gla::kMaxSortSeqs && units % 8 == 0) ? 1 : 0;
  prm.hs = nullptr;
  prm.slots = 0;
  return GLA_OK;
}

int launch_status(const char* fn, int rc, int dk, int dtype) {
  if (rc == -2) return fail(GLA_ERR_UNSUPPORTED, "%s: no kernel for dk=%d dtype=%d", fn, dk, dtype);
  if (rc != 0)
    return fail(GLA_ERR_LAUNCH, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
  return GLA_OK;
}

// Compute units of the current device (256 on MI355X; that value if no device answers).
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

// d_v slice of the bf16 forward: 64 or 128 columns per work item.  With 128 the
// gating of q and k and the score blocks serve twice the columns, but there are
// half as many work items to spread over the compute units.
//
// Rounds of ncu work items that `items` take, a last partial round weighted by
// how full it is (slice_model).
double slice_rounds(long long items, int ncu) {
  const long long full = items / ncu, rem = items - full * ncu;
  return (double)full +
         (rem ? gla::slice_model::kPartial + (1.0 - gla::slice_model::kPartial) * (double)rem / ncu : 0.0);
}

// d_v slice width (64 or 128) of the unsplit forward over `units` (sequence,
// head) pairs: 128 only for bf16 with dv a multiple of 128, and only where the
// slice model gives it the shorter time.
int slice_plan(long long units, int dv, int dtype, int ncu) {
  if (dtype != GLA_BF16 || dv <= 0 || dv % 128 != 0 || units <= 0 || ncu <= 0) return 64;
  const long long wide = units * (dv / 128);
  return gla::slice_model::kWide * slice_rounds(wide, ncu) < slice_rounds(2 * wide, ncu) ? 128 : 64;
}

// prm (filled by check_chunk_args with 64-column slices) switched to 128-column
// slices; the caller has checked bf16 and dv % 128 == 0.
void use_wide_slices(gla::ChunkParams& prm, long long units) {
  const long long items = units * (prm.DV / 128);
  prm.dvt = 128;
  prm.nvt = prm.DV / 128;
  prm.xcd_remap = (items % 8 == 0) ? 1 : 0;
}

void choose_slice(gla::ChunkParams& prm, long long units, int dtype) {
  if (slice_plan(units, prm.DV, dtype, device_cus()) == 128) use_wide_slices(prm, units);
}


// Sequence split of the backward: fixed-length bf16 inputs whose work items do
// not fill the device are cut into segments of at least kMinSegChunks chunks,
// about enough to give every compute unit one work item.  Returns the segment
// count (1 = none) and the segment length in tokens.
constexpr int kMinSegChunks = 8;

int split_plan(bool varlen, int dtype, long long items, int T, int& seg_len) {
  seg_len = T;
  if (varlen || dtype != GLA_BF16 || T <= 0) return 1;
  const int ncu = device_cus();
  if (items >= ncu) return 1;
  const int nch = (T + 63) / 64;
  long long want = (ncu + items - 1) / items;
  const long long by_len = nch / kMinSegChunks;
  long long nseg = want < by_len ? want : by_len;
  if (nseg < 2) return 1;
  const int seg_chunks = (int)((nch + nseg - 1) / nseg);
  seg_len = seg_chunks * 64;
  return (T + seg_len - 1) / seg_len;
}

// Segment plan of the forward (fixed-length bf16 inputs), from the split cost
// model of split_model.h: a split is considered only when the unsplit call's
// 64-column work items leave compute units idle (the page "Qwen Team Releases
// FlashQLA ...", section "Core Technical Principles": trigger when the device is
// clearly underused), and only for segment counts whose work items (128 columns
// of d_v when d_v allows) fit one wave.  Among those and the unsplit call it
// takes the least modelled time; ties keep fewer segments.  Returns the segment
// count (1 = unsplit) and the segment length in tokens (whole 64-token chunks).
int model_split_plan(bool varlen, int dtype, long long units, int dv, int T, int ncu, int& seg_len) {
  using namespace gla::split_model;
  seg_len = T;
  if (varlen || dtype != GLA_BF16 || T <= 0 || units <= 0 || dv <= 0 || dv % 64 != 0 || ncu <= 0)
    return 1;
  if (units * (dv / 64) >= ncu) return 1;
  const long long nch = ((long long)T + 63) / 64;
  const double t_unsplit = kMu1 * (double)nch + kMu0;   // one wave (the guard above)
  const long long items = units * ((dv % 128 == 0) ? dv / 128 : dv / 64);
  double best = t_unsplit;
  long long best_l = nch;
  for (long long n = 2; n <= nch && items * n <= ncu; ++n) {
    const long long l = (nch + n - 1) / n;    // chunks per segment
    const long long ns = (nch + l - 1) / l;   // segments that length gives
    const double t = kLambda1 * (double)l + kLambda2 * (double)ns + kLambda0;
    if (t < best) {
      best = t;
      best_l = l;
    }
  }
  if (best_l == nch) return 1;
  seg_len = (int)(best_l * 64);
  return (int)((nch + best_l - 1) / best_l);
}

int fwd_split_plan(bool varlen, int dtype, long long units, int dv, int T, int& seg_len) {
  return model_split_plan(varlen, dtype, units, dv, T, device_cus(), seg_len);
}

size_t split_bytes(long long units, int nseg, int dk, int dv) {
  const size_t st = (size_t)units * nseg * dk * dv * sizeof(float);
  const size_t dec = (size_t)units * nseg * dk * sizeof(float);
  return ((st + 255) / 256) * 256 + ((dec + 255) / 256) * 256;
}

// The backward runs d_v above 128 as column slices of 128 (the last one 64 when
// d_v is an odd multiple of 64), one launch each; dq, dk and dg are sums over the
// slices, kept in fp32 between launches: 3 x rows x dk floats.
int bwd_slices(int dv) { return (dv + 127) / 128; }
size_t bwd_partial_bytes(long long rows, int dk, int dv) {
  if (bwd_slices(dv) <= 1) return 0;
  return ((size_t)3 * rows * dk * sizeof(float) + 255) / 256 * 256;
}

// The three kernels of a split forward (prm filled by check_chunk_args; nseg > 1)
// with the segment states and decays in ws (split_bytes(...) bytes, 256-aligned).
int run_split(const char* fn, gla::ChunkParams& prm, long long units, int nseg, int seg_len,
              int dk, int dv, int dtype, const float* initial_state, float* final_state, char* ws,
              hipStream_t s) {
  const long long nblocks = units * nseg * prm.nvt;
  if (!fits_i32(nblocks)) return fail(GLA_ERR_INVALID_ARG, "%s: %lld work items", fn, nblocks);
  const size_t st_bytes = ((size_t)units * nseg * dk * dv * sizeof(float) + 255) / 256 * 256;
  prm.nseg = nseg;
  prm.seg_len = seg_len;
  prm.seg_state = reinterpret_cast<float*>(ws);
  prm.seg_decay = reinterpret_cast<float*>(ws + st_bytes);
  prm.xcd_remap = (nblocks % 8 == 0) ? 1 : 0;
  // 1. each segment's state from zero and its total decay
  int rc = gla::launch_chunk_fwd_pipe(prm, dk, true, (int)nblocks, s);
  if (rc != 0) return launch_status(fn, rc, dk, dtype);
  // 2. incoming state of every segment, and the final states
  gla::SegScanParams sp;
  sp.s0 = initial_state;
  sp.sT = final_state;
  sp.seg_state = prm.seg_state;
  sp.seg_decay = prm.seg_decay;
  sp.dk = dk;
  sp.dv = dv;
  sp.nseg = nseg;
  sp.reverse = 0;
  rc = gla::launch_seg_scan(sp, (int)units, s);
  if (rc != 0) return launch_status(fn, rc, dk, dtype);
  // 3. the forward pass of every segment from its incoming state
  rc = gla::launch_chunk_fwd_pipe(prm, dk, false, (int)nblocks, s);
  return launch_status(fn, rc, dk, dtype);
}

// Library-owned scratch of gla_chunk_fwd_noalloc: one copy per device, alive
// until the process ends.  In host code `scratch` only names the symbol; the
// device address comes from hipGetSymbolAddress, looked up once per device.
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];
static_assert(kNoallocScratchBytes == GLA_NOALLOC_SCRATCH_BYTES, "gla.h states the scratch size");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (nullptr with the message set).
void* scratch_for_current_device(const char* fn) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    fail(GLA_ERR_LAUNCH, "%s: no current HIP device (or device index >= %d)", fn, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      fail(GLA_ERR_LAUNCH, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", fn, dev,
           hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int gla_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                  const float* initial_state, void* o, float* final_state,
                  const int32_t* cu_seqlens, int num_seqs, int B, int H, int T, int dk,
                  int dv, int chunk_size, int dtype, void* stream) {
  g_last_error[0] = '\0';
  gla::ChunkParams prm;
  long long units = 0;
  bool nothing = false;
  const int st = check_chunk_args("gla_chunk_fwd", q, k, v, g, initial_state, o, final_state,
                                  cu_seqlens, num_seqs, B, H, T, dk, dv, chunk_size, dtype, prm,
                                  units, nothing);
  if (st != GLA_OK || nothing) return st;
  choose_slice(prm, units, dtype);
  const int rc = gla::launch_chunk_fwd(prm, dk, dtype, (int)(units * prm.nvt),
                                       reinterpret_cast<hipStream_t>(stream));
  return launch_status("gla_chunk_fwd", rc, dk, dtype);
}

size_t gla_chunk_fwd_workspace_size(int num_seqs, int B, int H, int T, int dk, int dv,
                                    int chunk_size, int dtype) {
  if (B <= 0 || H <= 0 || T <= 0 || dk <= 0 || dv <= 0 || chunk_size != 64) return 0;
  if (dv % 64 != 0) return 0;
  const long long units = (long long)B * H;
  int seg_len = 0;
  const int nseg = fwd_split_plan(num_seqs > 0, dtype, units, dv, T, seg_len);
  return nseg > 1 ? split_bytes(units, nseg, dk, dv) : 0;
}

int gla_chunk_fwd_ws(const void* q, const void* k, const void* v, const void* g,
                     const float* initial_state, void* o, float* final_state,
                     const int32_t* cu_seqlens, int num_seqs, int B, int H, int T, int dk,
                     int dv, int chunk_size, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  gla::ChunkParams prm;
  long long units = 0;
  bool nothing = false;
  const int st = check_chunk_args("gla_chunk_fwd_ws", q, k, v, g, initial_state, o, final_state,
                                  cu_seqlens, num_seqs, B, H, T, dk, dv, chunk_size, dtype, prm,
                                  units, nothing);
  if (st != GLA_OK || nothing) return st;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int seg_len = T;
  const int nseg = fwd_split_plan(cu_seqlens != nullptr, dtype, units, dv, T, seg_len);
  if (nseg == 1) {
    choose_slice(prm, units, dtype);
    const int rc = gla::launch_chunk_fwd(prm, dk, dtype, (int)(units * prm.nvt), s);
    return launch_status("gla_chunk_fwd_ws", rc, dk, dtype);
  }
  if (dtype == GLA_BF16 && dv % 128 == 0) {   // split work items take the 128-column slice
    prm.dvt = 128;
    prm.nvt = dv / 128;
  }
  const size_t need = split_bytes(units, nseg, dk, dv);
  if (!workspace || workspace_bytes < need)
    return fail(GLA_ERR_INVALID_ARG, "gla_chunk_fwd_ws: workspace of %zu bytes given, %zu needed",
                workspace ? workspace_bytes : (size_t)0, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(GLA_ERR_INVALID_ARG, "gla_chunk_fwd_ws: workspace is not 256-byte aligned");
  return run_split("gla_chunk_fwd_ws", prm, units, nseg, seg_len, dk, dv, dtype, initial_state,
                   final_state, static_cast<char*>(workspace), s);
}

int gla_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* g,
                          const float* initial_state, void* o, float* final_state,
                          const int32_t* cu_seqlens, int num_seqs, int B, int H, int T, int dk,
                          int dv, int chunk_size, int dtype, void* stream) {
  g_last_error[0] = '\0';
  const char* fn = "gla_chunk_fwd_noalloc";
  gla::ChunkParams prm;
  long long units = 0;
  bool nothing = false;
  const int st = check_chunk_args(fn, q, k, v, g, initial_state, o, final_state, cu_seqlens,
                                  num_seqs, B, H, T, dk, dv, chunk_size, dtype, prm, units, nothing);
  if (st != GLA_OK || nothing) return st;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int seg_len = T;
  const int nseg = fwd_split_plan(cu_seqlens != nullptr, dtype, units, dv, T, seg_len);
  if (nseg == 1) {   // no scratch needed: the plain forward
    choose_slice(prm, units, dtype);
    const int rc = gla::launch_chunk_fwd(prm, dk, dtype, (int)(units * prm.nvt), s);
    return launch_status(fn, rc, dk, dtype);
  }
  if (dtype == GLA_BF16 && dv % 128 == 0) {   // as in gla_chunk_fwd_ws
    prm.dvt = 128;
    prm.nvt = dv / 128;
  }
  const size_t need = split_bytes(units, nseg, dk, dv);
  if (need > kNoallocScratchBytes)
    return fail(GLA_ERR_INVALID_ARG,
                "%s: this shape's sequence split needs %zu bytes of scratch, more than the %zu of "
                "the library's scratch array; use gla_chunk_fwd_ws with a workspace",
                fn, need, kNoallocScratchBytes);
  char* ws = static_cast<char*>(scratch_for_current_device(fn));
  if (!ws) return GLA_ERR_LAUNCH;
  return run_split(fn, prm, units, nseg, seg_len, dk, dv, dtype, initial_state, final_state, ws, s);
}

int gla_chunk_fwd_sliced(const void* q, const void* k, const void* v, const void* g,
                         const float* initial_state, void* o, float* final_state,
                         const int32_t* cu_seqlens, int num_seqs, int B, int H, int T, int dk,
                         int dv, int chunk_size, int dtype, int dv_slice, void* stream) {
  g_last_error[0] = '\0';
  const char* fn = "gla_chunk_fwd_sliced";
  if (dv_slice != 0 && dv_slice != 64 && dv_slice != 128)
    return fail(GLA_ERR_INVALID_ARG, "%s: dv_slice = %d (0, 64 or 128)", fn, dv_slice);
  gla::ChunkParams prm;
  long long units = 0;
  bool nothing = false;
  const int st = check_chunk_args(fn, q, k, v, g, initial_state, o, final_state, cu_seqlens,
                                  num_seqs, B, H, T, dk, dv, chunk_size, dtype, prm, units, nothing);
  if (st != GLA_OK) return st;
  if (dv_slice == 128 && (dtype != GLA_BF16 || dv % 128 != 0))
    return fail(GLA_ERR_UNSUPPORTED, "%s: 128-column slices need bf16 and dv a multiple of 128 (dtype=%d dv=%d)",
                fn, dtype, dv);
  if (nothing) return GLA_OK;
  const int width = dv_slice ? dv_slice : slice_plan(units, dv, dtype, device_cus());
  if (width == 128) use_wide_slices(prm, units);
  const int rc = gla::launch_chunk_fwd(prm, dk, dtype, (int)(units * prm.nvt),
                                       reinterpret_cast<hipStream_t>(stream));
  return launch_status(fn, rc, dk, dtype);
}

int gla_slice_plan(long long units, int dv, int dtype, int num_cus) {
  return slice_plan(units, dv, dtype, num_cus);
}

int gla_split_plan(long long units, int T, int dv, int dtype, int num_cus, int* seg_len) {
  int len = T;
  const int n = model_split_plan(false, dtype, units, dv, T, num_cus, len);
  if (seg_len) *seg_len = len;
  return n;
}

namespace {
// segment length (whole chunks) and count for a caller-chosen segment count
int forced_plan(int T, int num_segments, int& seg_len) {
  const long long nch = ((long long)T + 63) / 64;
  const long long l = (nch + num_segments - 1) / num_segments;
  seg_len = (int)(l * 64);
  return (int)((nch + l - 1) / l);
}
}  // namespace

size_t gla_chunk_fwd_segments_workspace_size(int B, int H, int T, int dk, int dv, int num_segments) {
  if (B <= 0 || H <= 0 || T <= 0 || dk <= 0 || dv <= 0 || num_segments < 1) return 0;
  const long long nch = ((long long)T + 63) / 64;
  if (num_segments > nch) return 0;
  int seg_len = 0;
  const int nseg = forced_plan(T, num_segments, seg_len);
  return nseg > 1 ? split_bytes((long long)B * H, nseg, dk, dv) : 0;
}

int gla_chunk_fwd_segments(const void* q, const void* k, const void* v, const void* g,
                           const float* initial_state, void* o, float* final_state, int B, int H,
                           int T, int dk, int dv, int chunk_size, int dtype, int num_segments,
                           void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  const char* fn = "gla_chunk_fwd_segments";
  gla::ChunkParams prm;
  long long units = 0;
  bool nothing = false;
  const int st = check_chunk_args(fn, q, k, v, g, initial_state, o, final_state, nullptr, 0, B, H, T,
                                  dk, dv, chunk_size, dtype, prm, units, nothing);
  if (st != GLA_OK || nothing) return st;
  const long long nch = ((long long)T + 63) / 64;
  if (num_segments < 1 || num_segments > nch)
    return fail(GLA_ERR_INVALID_ARG, "%s: num_segments = %d, must be in [1, %lld] (one chunk or more each)",
                fn, num_segments, nch);
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int seg_len = T;
  const int nseg = forced_plan(T, num_segments, seg_len);
  if (nseg == 1) {
    choose_slice(prm, units, dtype);
    const int rc = gla::launch_chunk_fwd(prm, dk, dtype, (int)(units * prm.nvt), s);
    return launch_status(fn, rc, dk, dtype);
  }
  if (dtype != GLA_BF16)
    return fail(GLA_ERR_UNSUPPORTED, "%s: the sequence split runs on bf16 inputs only", fn);
  if (dv % 128 == 0) {   // split work items take the 128-column slice, as in gla_chunk_fwd_ws
    prm.dvt = 128;
    prm.nvt = dv / 128;
  }
  const size_t need = split_bytes(units, nseg, dk, dv);
  if (!workspace || workspace_bytes < need)
    return fail(GLA_ERR_INVALID_ARG, "%s: workspace of %zu bytes given, %zu needed", fn,
                workspace ? workspace_bytes : (size_t)0, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(GLA_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);
  return run_split(fn, prm, units, nseg, seg_len, dk, dv, dtype, initial_state, final_state,
                   static_cast<char*>(workspace), s);
}

size_t gla_chunk_bwd_workspace_size(int num_seqs, int B, int H, int T, int dk, int dv,
                                    int chunk_size, int dtype) {
  if (dtype != GLA_BF16 || chunk_size != 64 || B <= 0 || H <= 0 || T < 0) return 0;
  if ((dk != 64 && dk != 128) || dv <= 0 || dv % 64 != 0) return 0;
  const long long nseq = num_seqs > 0 ? num_seqs : B;
  const long long tokens = num_seqs > 0 ? (long long)T : (long long)B * T;
  const long long slots = nseq + tokens / 64 + 1;
  const size_t states = ((size_t)H * slots * dk * dv * 2 + 255) / 256 * 256;
  int seg_len = T;
  const int nseg = split_plan(num_seqs > 0, dtype, nseq * H, T, seg_len);
  return states + (nseg > 1 ? split_bytes(nseq * H, nseg, dk, dv) : 0) + bwd_partial_bytes(H * tokens, dk, dv);
}

}  // extern "C"

namespace {

// gla_chunk_bwd, and gla_chunk_bwd_saved (states_ready: the workspace already
// holds the chunk states, written by gla_chunk_fwd_states)
int chunk_bwd_impl(const char* fn, bool states_ready, const void* q, const void* k, const void* v,
                   const void* g, const float* initial_state, const void* d_o,
                   const float* d_final_state, void* d_q, void* d_k, void* d_v, void* d_g,
                   float* d_initial_state, const int32_t* cu_seqlens, int num_seqs, int B, int H,
                   int T, int dk, int dv, int chunk_size, int dtype, void* workspace,
                   size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  if (dtype != GLA_BF16 && dtype != GLA_F32)
    return fail(GLA_ERR_INVALID_ARG, "%s: dtype %d is not GLA_BF16 or GLA_F32", fn, dtype);
  if (dtype != GLA_BF16)
    return fail(GLA_ERR_UNSUPPORTED, "%s: only GLA_BF16 is implemented", fn);
  if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0)
    return fail(GLA_ERR_INVALID_ARG, "%s: B=%d H=%d T=%d dk=%d dv=%d must be positive (T >= 0)", fn,
                B, H, T, dk, dv);
  if (chunk_size != 64)
    return fail(GLA_ERR_UNSUPPORTED, "%s: chunk_size %d (only 64 is implemented)", fn, chunk_size);
  if ((dk != 64 && dk != 128) || dv % 64 != 0)
    return fail(GLA_ERR_UNSUPPORTED, "%s: dk=%d dv=%d (dk must be 64 or 128, dv a multiple of 64)", fn, dk,
                dv);
  int nseq = B;
  if (cu_seqlens) {
    if (B != 1)
      return fail(GLA_ERR_INVALID_ARG, "%s: packed sequences (cu_seqlens) need B == 1, got %d", fn, B);
    if (num_seqs <= 0)
      return fail(GLA_ERR_INVALID_ARG, "%s: num_seqs=%d must be positive with cu_seqlens", fn, num_seqs);
    nseq = num_seqs;
  }
  if (!fits_i32((long long)B * H * T * dk) || !fits_i32((long long)B * H * T * dv) ||
      !fits_i32((long long)nseq * H * dk * dv))
    return fail(GLA_ERR_INVALID_ARG, "%s: tensor sizes exceed int32 indexing", fn);
  // one sequence's chunk states are addressed with 32-bit byte offsets
  if (!fits_i32(((long long)T / 64 + 1) * dk * dv * 2))
    return fail(GLA_ERR_INVALID_ARG, "%s: T=%d is too long for one call's chunk states", fn, T);
  const bool any_tokens = (long long)B * H * T > 0;
  if (any_tokens && (!q || !k || !v || !g || !d_o || !d_q || !d_k || !d_v || !d_g))
    return fail(GLA_ERR_INVALID_ARG, "%s: q, k, v, g, d_o, d_q, d_k, d_v and d_g must be non-null", fn);
  const void* ptrs[] = {q, k, v, g, d_o, d_q, d_k, d_v, d_g, initial_state, d_final_state,
                        d_initial_state, cu_seqlens};
  const char* names[] = {"q", "k", "v", "g", "d_o", "d_q", "d_k", "d_v", "d_g", "initial_state",
                         "d_final_state", "d_initial_state", "cu_seqlens"};
  for (int i = 0; i < 13; ++i)
    if (ptrs[i] && !aligned16(ptrs[i]))
      return fail(GLA_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, names[i]);
  if (!any_tokens && !d_initial_state) return GLA_OK;
  const size_t need = gla_chunk_bwd_workspace_size(cu_seqlens ? num_seqs : 0, B, H, T, dk, dv,
                                                   chunk_size, dtype);
  if (!workspace || workspace_bytes < need)
    return fail(GLA_ERR_INVALID_ARG, "%s: workspace of %zu bytes given, %zu needed", fn,
                workspace ? workspace_bytes : (size_t)0, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(GLA_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);
  const long long units = (long long)nseq * H;
  const int nvt = dv / 64;
  if (!fits_i32(units * nvt))
    return fail(GLA_ERR_INVALID_ARG, "%s: %lld work items", fn, units * nvt);
  const long long tokens = cu_seqlens ? (long long)T : (long long)B * T;

  gla::BwdParams prm;
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.g = g;
  prm.dout = d_o;
  prm.s0 = initial_state;
  prm.dsT = d_final_state;
  prm.dq = d_q;
  prm.dk = d_k;
  prm.dv = d_v;
  prm.dg = d_g;
  prm.ds0 = d_initial_state;
  prm.hs = static_cast<unsigned short*>(workspace);
  prm.cu = cu_seqlens;
  prm.H = H;
  prm.T = T;
  prm.DV = dv;
  prm.nvt = nvt;
  prm.slots = (int)(nseq + tokens / 64 + 1);
  prm.ldv = dv;
  prm.col0 = 0;
  prm.pmode = 0;
  prm.part = nullptr;
  prm.part_rows = (long)(H * tokens);
  prm.xcd_remap = ((units * nvt) % 8 == 0) ? 1 : 0;
  // sequence split: as in the forward, fixed-length sequences of too few units
  // to fill the device are cut into segments of whole chunks
  int seg_len = T;
  const int nseg = split_plan(cu_seqlens != nullptr, dtype, units, T, seg_len);
  prm.nseg = nseg;
  prm.seg_len = nseg > 1 ? seg_len : (T > 0 ? (T + 63) / 64 * 64 : 64);
  if (cu_seqlens) prm.seg_len = 1 << 30;   // one segment whatever the packed lengths
  prm.seg_state = nullptr;
  prm.seg_decay = nullptr;
  const size_t states_bytes = ((size_t)H * prm.slots * dk * dv * 2 + 255) / 256 * 256;
  if (nseg > 1) {
    char* const sp = static_cast<char*>(workspace) + states_bytes;
    const size_t st_bytes = ((size_t)units * nseg * dk * dv * sizeof(float) + 255) / 256 * 256;
    prm.seg_state = reinterpret_cast<float*>(sp);
    prm.seg_decay = reinterpret_cast<float*>(sp + st_bytes);
  }
  if (bwd_slices(dv) > 1)
    prm.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + states_bytes +
                                        (nseg > 1 ? split_bytes(units, nseg, dk, dv) : 0));
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // 1. the state entering every chunk: the forward's pipelined kernel, states only
  gla::ChunkParams fp;
  fp.q = q;
  fp.k = k;
  fp.v = v;
  fp.g = g;
  fp.s0 = initial_state;
  fp.o = nullptr;
  fp.sT = nullptr;
  fp.cu = cu_seqlens;
  fp.H = H;
  fp.T = T;
  fp.DV = dv;
  fp.dvt = 64;
  fp.nvt = nvt;
  fp.xcd_remap = ((units * nvt) % 8 == 0) ? 1 : 0;
  fp.nseg = 1;
  fp.seg_len = T;
  fp.nseq = nseq;
  // packed sequences: the longest units' work items first, as in the forward
  fp.sort_units = (cu_seqlens && nseq <= gla::kMaxSortSeqs && units % 8 == 0) ? 1 : 0;
  fp.seg_state = nullptr;
  fp.seg_decay = nullptr;
  fp.hs = prm.hs;
  fp.slots = prm.slots;
  int rc = states_ready ? 0 : gla::launch_chunk_fwd_states(fp, dk, (int)(units * nvt), s);
  if (rc != 0) return launch_status(fn, rc, dk, dtype);
  if (nseg > 1) {
    // 2. each later segment's own state gradient and decay, 3. every segment's
    //    incoming state gradient (segments last to first, from d_final_state)
    const long long nb2 = units * (nseg - 1) * nvt;
    if (!fits_i32(nb2) || !fits_i32(units * nseg))
      return fail(GLA_ERR_INVALID_ARG, "%s: %lld work items", fn, nb2);
    // the pipelined kernel again, chunks last to first, q and dO in the key and
    // value places, B = 0 at each segment's end
    gla::ChunkParams gp = fp;
    gp.k = q;
    gp.v = d_o;
    gp.s0 = nullptr;
    gp.hs = nullptr;
    gp.nseg = nseg;
    gp.seg_len = seg_len;
    gp.seg_state = prm.seg_state;
    gp.seg_decay = prm.seg_decay;
    gp.xcd_remap = (nb2 % 8 == 0) ? 1 : 0;
    rc = gla::launch_chunk_seg_grad(gp, dk, (int)nb2, s);
    if (rc != 0) return launch_status(fn, rc, dk, dtype);
    gla::SegScanParams sp;
    sp.s0 = d_final_state;
    sp.sT = nullptr;
    sp.seg_state = prm.seg_state;
    sp.seg_decay = prm.seg_decay;
    sp.dk = dk;
    sp.dv = dv;
    sp.nseg = nseg;
    sp.reverse = 1;
    rc = gla::launch_seg_scan(sp, (int)units, s);
    if (rc != 0) return launch_status(fn, rc, dk, dtype);
  }
  // 4. the gradients chunk by chunk, last to first, per (unit, segment); d_v above
  //    128 one column slice per launch, in order on the stream, dq, dk and dg summed
  const int nsl = bwd_slices(dv);
  for (int sl = 0; sl < nsl; ++sl) {
    prm.col0 = 128 * sl;
    prm.pmode = nsl == 1 ? 0 : sl == 0 ? 1 : sl == nsl - 1 ? 3 : 2;
    rc = gla::launch_chunk_bwd(prm, dk, dv - prm.col0 >= 128 ? 128 : 64, (int)(units * nseg), s);
    if (rc != 0) break;
  }
  return launch_status(fn, rc, dk, dtype);
}

}  // namespace

extern "C" {

int gla_chunk_bwd(const void* q, const void* k, const void* v, const void* g,
                  const float* initial_state, const void* d_o, const float* d_final_state,
                  void* d_q, void* d_k, void* d_v, void* d_g, float* d_initial_state,
                  const int32_t* cu_seqlens, int num_seqs, int B, int H, int T, int dk, int dv,
                  int chunk_size, int dtype, void* workspace, size_t workspace_bytes,
                  void* stream) {
  return chunk_bwd_impl("gla_chunk_bwd", false, q, k, v, g, initial_state, d_o, d_final_state, d_q, d_k,
                        d_v, d_g, d_initial_state, cu_seqlens, num_seqs, B, H, T, dk, dv, chunk_size,
                        dtype, workspace, workspace_bytes, stream);
}

int gla_chunk_bwd_saved(const void* q, const void* k, const void* v, const void* g,
                        const float* initial_state, const void* d_o, const float* d_final_state,
                        void* d_q, void* d_k, void* d_v, void* d_g, float* d_initial_state,
                        const int32_t* cu_seqlens, int num_seqs, int B, int H, int T, int dk, int dv,
                        int chunk_size, int dtype, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return chunk_bwd_impl("gla_chunk_bwd_saved", true, q, k, v, g, initial_state, d_o, d_final_state, d_q,
                        d_k, d_v, d_g, d_initial_state, cu_seqlens, num_seqs, B, H, T, dk, dv,
                        chunk_size, dtype, workspace, workspace_bytes, stream);
}

int gla_chunk_fwd_states(const void* q, const void* k, const void* v, const void* g,
                         const float* initial_state, void* o, float* final_state,
                         const int32_t* cu_seqlens, int num_seqs, int B, int H, int T, int dk,
                         int dv, int chunk_size, int dtype, void* chunk_states,
                         size_t chunk_states_bytes, void* stream) {
  g_last_error[0] = '\0';
  const char* fn = "gla_chunk_fwd_states";
  gla::ChunkParams prm;
  long long units = 0;
  bool nothing = false;
  const int st = check_chunk_args(fn, q, k, v, g, initial_state, o, final_state, cu_seqlens, num_seqs,
                                  B, H, T, dk, dv, chunk_size, dtype, prm, units, nothing);
  if (st != GLA_OK) return st;
  if (dtype != GLA_BF16)
    return fail(GLA_ERR_UNSUPPORTED, "%s: chunk states come from the bf16 path only", fn);
  if ((dk != 64 && dk != 128) || dv % 64 != 0)
    return fail(GLA_ERR_UNSUPPORTED, "%s: dk=%d dv=%d (as for gla_chunk_bwd: dk 64 or 128, dv a multiple of 64)",
                fn, dk, dv);
  if (!fits_i32(((long long)T / 64 + 1) * dk * dv * 2))
    return fail(GLA_ERR_INVALID_ARG, "%s: T=%d is too long for one call's chunk states", fn, T);
  if (nothing) return GLA_OK;
  const size_t need = gla_chunk_bwd_workspace_size(cu_seqlens ? num_seqs : 0, B, H, T, dk, dv,
                                                   chunk_size, dtype);
  if (!chunk_states || chunk_states_bytes < need)
    return fail(GLA_ERR_INVALID_ARG, "%s: chunk_states of %zu bytes given, %zu needed", fn,
                chunk_states ? chunk_states_bytes : (size_t)0, need);
  if ((reinterpret_cast<uintptr_t>(chunk_states) & 255u) != 0)
    return fail(GLA_ERR_INVALID_ARG, "%s: chunk_states is not 256-byte aligned", fn);
  const long long nseq = cu_seqlens ? num_seqs : B;
  const long long tokens = cu_seqlens ? (long long)T : (long long)B * T;
  // the backward's layout: 64-column slices, one run over every sequence
  prm.dvt = 64;
  prm.nvt = dv / 64;
  prm.hs = static_cast<unsigned short*>(chunk_states);
  prm.slots = (int)(nseq + tokens / 64 + 1);
  const int rc = gla::launch_chunk_fwd_full_states(prm, dk, (int)(units * prm.nvt),
                                                   reinterpret_cast<hipStream_t>(stream));
  return launch_status(fn, rc, dk, dtype);
}

int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                  const float* initial_state, void* o, float* final_state, const int32_t* cu_seqlens,
                  int num_seqs, int B, int H, int T, int dk, int dv, int chunk_size, int dtype,
                  void* stream) {
  g_last_error[0] = '\0';
  const char* fn = "gdn_chunk_fwd";
  if (dtype != GLA_BF16 && dtype != GLA_F32)
    return fail(GLA_ERR_INVALID_ARG, "%s: dtype %d is not GLA_BF16 or GLA_F32", fn, dtype);
  if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0)
    return fail(GLA_ERR_INVALID_ARG, "%s: B=%d H=%d T=%d dk=%d dv=%d must be positive (T >= 0)", fn,
                B, H, T, dk, dv);
  if (dtype != GLA_BF16)
    return fail(GLA_ERR_UNSUPPORTED, "%s: only GLA_BF16 is implemented", fn);
  if (chunk_size != 64)
    return fail(GLA_ERR_UNSUPPORTED, "%s: chunk_size %d (only 64 is implemented)", fn, chunk_size);
  if (dk != 64 && dk != 128)
    return fail(GLA_ERR_UNSUPPORTED, "%s: dk=%d (64 or 128)", fn, dk);
  if (dv % 64 != 0 || dv > 512)
    return fail(GLA_ERR_UNSUPPORTED, "%s: dv=%d must be a multiple of 64 up to 512", fn, dv);
  int nseq = B;
  if (cu_seqlens) {
    if (B != 1)
      return fail(GLA_ERR_INVALID_ARG, "%s: packed sequences (cu_seqlens) need B == 1, got %d", fn, B);
    if (num_seqs <= 0)
      return fail(GLA_ERR_INVALID_ARG, "%s: num_seqs=%d must be positive with cu_seqlens", fn,
                  num_seqs);
    nseq = num_seqs;
  }
  if (!fits_i32((long long)B * H * T * dv) || !fits_i32((long long)B * H * T * dk) ||
      !fits_i32((long long)nseq * H * dk * dv))
    return fail(GLA_ERR_INVALID_ARG, "%s: tensor sizes exceed int32 indexing", fn);
  const bool any_tokens = (long long)B * H * T > 0;
  if (any_tokens && (!q || !k || !v || !g || !beta || !o))
    return fail(GLA_ERR_INVALID_ARG, "%s: q, k, v, g, beta and o must be non-null", fn);
  const void* ptrs[] = {q, k, v, o, initial_state, final_state, cu_seqlens};
  const char* names[] = {"q", "k", "v", "o", "initial_state", "final_state", "cu_seqlens"};
  for (int i = 0; i < 7; ++i)
    if (ptrs[i] && !aligned16(ptrs[i]))
      return fail(GLA_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, names[i]);
  if ((g && (reinterpret_cast<uintptr_t>(g) & 3u)) || (beta && (reinterpret_cast<uintptr_t>(beta) & 3u)))
    return fail(GLA_ERR_INVALID_ARG, "%s: g and beta must be 4-byte aligned", fn);
  const long long units = (long long)nseq * H;
  const int nvt = dv / 64;
  const long long nblocks = units * nvt;
  if (!fits_i32(nblocks))
    return fail(GLA_ERR_INVALID_ARG, "%s: %lld work items", fn, nblocks);
  if (!any_tokens && !final_state) return GLA_OK;
  gla::GdnParams prm;
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.g = g;
  prm.beta = beta;
  prm.s0 = initial_state;
  prm.o = o;
  prm.sT = final_state;
  prm.cu = cu_seqlens;
  prm.H = H;
  prm.T = T;
  prm.DV = dv;
  prm.nvt = nvt;
  prm.xcd_remap = (nblocks % 8 == 0) ? 1 : 0;
  const int rc = gla::launch_gdn_chunk_fwd(prm, dk, (int)nblocks, reinterpret_cast<hipStream_t>(stream));
  return launch_status(fn, rc, dk, dtype);
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
