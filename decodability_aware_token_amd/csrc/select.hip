// Budgeted selection (target token selection): keep the k_r masked tokens of each request with
// the largest importance delta.  Project page "FOCUS: DLLMs Know How to Tame Their Compute
// Bound", cards "Design" (adaptive budget over likely-decodable candidates) and "Runtime
// Action" (dynamic budgeting, token eviction).
//
// One wavefront per request (the selection itself is select_request in select_impl.h).
#include "select_impl.h"

namespace focus {
namespace {

__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= a.B) return;  // uniform per wave
  const SelectInputs in = select_inputs(a, r, lane);
  const float dj = lane < a.blk ? a.delta[(size_t)r * a.blk + lane] : 0.f;
  select_request(a, r, in, dj, lane);
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3((a.B + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace focus
