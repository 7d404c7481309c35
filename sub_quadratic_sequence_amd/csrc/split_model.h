// Fitted constants of the forward's cost models: the sequence split
// (microseconds) and the d_v slice width (ratios).
//
// The page "Qwen Team Releases FlashQLA for High-Performance Linear Attention",
// section "Core Technical Principles", models a split in its "one wave" case:
// the per-segment passes (the state pass and the forward from the incoming
// states) take time proportional to the chunks per segment L, the scan across
// segments time proportional to the segment count N / L, so
// T = lambda_1 L + lambda_2 N / L, with the lambdas tuned on the hardware.  Here
// the split call also has a fixed cost lambda_0, and the unsplit call takes
// mu_1 N w + mu_0 for N chunks and w waves of its work items.
//
// Values: least-squares fits to times measured on one MI355X (256 CUs) by
//   python -m sub_quadratic_sequence_amd.fit_split
// on bf16 inputs with d_k = d_v = 128: 214 split timings (gla_chunk_fwd_segments,
// units = B x H in 1 .. 64, T in 1024 .. 65536, up to one wave of 128-column work
// items) and 27 unsplit ones; relative residuals, median / max: split 7.8% / 28%,
// unsplit 4.2% / 9.4%.  On that grid the plan this model picks runs on average
// 1.2% (at most 8%) slower than the fastest measured segment count.
#pragma once

namespace gla {
namespace split_model {

constexpr double kLambda1 = 5.35;  // per chunk of segment length, one wave of work items
constexpr double kLambda2 = 0.450; // per segment
constexpr double kLambda0 = 22.6;  // per split call
constexpr double kMu1 = 2.13;      // per chunk and wave of the unsplit call
constexpr double kMu0 = 10.8;      // per unsplit call

}  // namespace split_model

// d_v slice width of the unsplit bf16 forward: 64 or 128 value columns per work
// item (one workgroup that holds a compute unit for its whole sequence).  A call
// runs in rounds of num_cus work items.  A last, partial round with a fraction f
// of the compute units busy costs kPartial + (1 - kPartial) f of a full round,
// and a round of 128-column items costs kWide rounds of 64-column items (twice
// the columns per item, the gating of q and k shared by them).  The 128-column
// slice is taken when kWide x rounds(items at 128) < rounds(items at 64).
//
// Values: from 115 pairs of timings of both widths on one MI355X (256 CUs), taken by
//   python -m sub_quadratic_sequence_amd.fit_slice
// (bf16, d_k = 128, d_v in {128, 256}, units = B x H from 32 to 800, T from 512
// to 8192).  Searched on a 0.05 grid, the (kWide, kPartial) pairs whose choices
// lose least form a band from (1.5, 1.0) to (1.95, 0.1); (1.8, 0.5) lies in it.  Its choices run on
// average 0.4% slower than the faster width at each point (5% at most, except
// one 80-item point at 20%), against 3.9% (at most 28%) for the threshold
// "128 columns once their work items fill the device".  A second run of the
// script on another MI355X put the least loss at (1.9, 0.15): 0.23% on average,
// against 0.27% for (1.8, 0.5) and 4.0% for the threshold.
namespace slice_model {

constexpr double kWide = 1.8;
constexpr double kPartial = 0.5;

}  // namespace slice_model
}  // namespace gla
