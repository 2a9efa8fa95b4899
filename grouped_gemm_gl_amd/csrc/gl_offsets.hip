// Split-offset scan kernel: one workgroup runs offsets_block (gl_offsets.hpp).
#include "gl_offsets.hpp"

namespace gl {

__global__ __launch_bounds__(kScanThreads) void offsets_kernel(const int64_t *__restrict__ m_splits, int G,
                                                               int64_t total_rows, void *ws, int split_slots) {
  offsets_block<kScanThreads>(m_splits, G, total_rows, ws, split_slots);
}

// split_slots: partial-tile slots of the workspace's split area (kSplitSlots for a
// workspace of gl_workspace_size)
hipError_t launch_offsets(const int64_t *m_splits, int G, int64_t total_rows, void *ws, int split_slots,
                          hipStream_t stream) {
  hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(kScanThreads), 0, stream, m_splits, G, total_rows, ws,
                     split_slots);
  return hipGetLastError();
}

}  // namespace gl
