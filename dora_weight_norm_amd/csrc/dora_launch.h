// Kernel launchers behind the C ABI (host side, defined in the .hip files).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dora_plan.h"

namespace dora {

// Timing marks of one norm call: ev[0] is recorded on the stream before the
// call's first launch and ev[i] after its i-th launch, for i < n; null
// entries are skipped. Lives on the caller's stack for one call.
struct Marks {
  const hipEvent_t* ev;
  int n;
  int next;
};
constexpr int kMaxLaunchEvents = 8;

hipError_t launch_norm_factored(const NormPlan& p, const void* W, const void* A, const void* B, void* ws,
                                float s, const float* m, float eps, float* wnorm, float* g, hipStream_t st,
                                const hipEvent_t* events, int n_events);
hipError_t launch_norm_dense(const NormPlan& p, const void* W, const void* A, const void* B, void* ws, float s,
                             const float* m, float eps, float* wnorm, float* g, hipStream_t st,
                             const hipEvent_t* events, int n_events);
hipError_t launch_norm_rowonly(const void* W, int dtype, int64_t d_out, int64_t d_in, bool vec, const float* m,
                               float eps, float* wnorm, float* g, hipStream_t st, const hipEvent_t* events,
                               int n_events);
hipError_t launch_magnitude(const float* m, const float* wnorm, float eps, int64_t n, float* g, hipStream_t st);
hipError_t launch_cast(const float* wnorm, int64_t n, int dtype, void* out, hipStream_t st);
hipError_t launch_compose(const void* base, const void* lora, const float* g, float s, int dtype, int64_t T,
                          int64_t d_out, void* out, bool vec, bool add_base, hipStream_t st);
size_t compose_bwd_workspace_bytes(int64_t T, int64_t d_out);
hipError_t launch_compose_bwd(const void* dy, const void* base, const void* lora, const float* g, float s, int dtype,
                              int64_t T, int64_t d_out, void* d_base, void* d_lora, float* dg, const float* wnorm,
                              float eps, float* dm, void* ws, bool vec, hipStream_t st);
size_t fast_kernel_lds_bytes(int cfg);
size_t gen_kernel_lds_bytes(int cfg);

}  // namespace dora
