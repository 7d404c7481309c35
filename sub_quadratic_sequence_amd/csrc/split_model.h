// Fitted constants of the forward's sequence-split cost model (microseconds).
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
}  // namespace gla
