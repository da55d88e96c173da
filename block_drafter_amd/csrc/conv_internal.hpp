// Internal interface of DFlash2's dynamic grouped convolution kernels (conv.hip).
#pragma once
#include "dspine_internal.hpp"

namespace dspine {

// One branch's convolution over B request blocks of W rows (row m = b*W + i).
// delta [M, 4G] holds W_delta X with columns (side*2 + tap)*G + g; base [4, H]
// (model dtype) rows side*2 + tap.
struct ConvParams {
  int32_t M, W, H, G, cg;         // rows, block width, hidden, groups, group width
  const float* delta;
  const void* base;
  // prepare (side 0): X = x * rsqrt(S/H + eps) * gain, S the row's sum of
  // squares from `lists` statistics lists of stride ld; output act [M, H]
  // in the GEMM operand type
  const float* x;
  const float* stats;
  int32_t lists, ld;
  const void* gain;
  float eps;
  void* act;
  // finish (side 1): x_out += Conv_1(o); stats_out[m] = sum of squares of the new row
  const float* o;
  float* x_out;
  float* stats_out;
};
hipError_t launch_conv_prepare(const ConvParams& p, int dtype, hipStream_t s);
hipError_t launch_conv_finish(const ConvParams& p, int dtype, hipStream_t s);

}  // namespace dspine
