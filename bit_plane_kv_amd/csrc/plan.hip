// Per-head plan kernel (the plan itself, and its sources, are in plan_device.h) and the
// fixed-depth comparator plan.
#include "plan_device.h"

namespace fathom {
namespace {

// zero (if given): the head's G per-row counters are cleared, for a later kernel of the
// same step that counts its workgroups per row.
__global__ __launch_bounds__(256) void k_plan(const float *__restrict__ q,
                                              const float *__restrict__ var, int G, int B,
                                              uint8_t *__restrict__ depth,
                                              uint32_t *__restrict__ zero) {
    __shared__ int cnt[kD];
    const int h = blockIdx.x, tid = threadIdx.x;
    if (zero && tid < G) zero[(size_t)h * G + tid] = 0u;
    float qp[FATHOM_MAX_G], vp;
    plan_load<256>(q, var, G, h, qp, vp);
    plan_from<256>(qp, vp, G, B, cnt);
    if (tid < kD) depth[(size_t)h * kD + tid] = (uint8_t)cnt[tid];
}

// Fixed comparator plan: depth 4 on the n_channels channels of largest var (equal var:
// lower channel index).  Rank by counting; 128 threads.
__global__ __launch_bounds__(128) void k_plan_fixed(const float *__restrict__ var,
                                                    int n_channels,
                                                    uint8_t *__restrict__ depth) {
    __shared__ float v[kD];
    const int h = blockIdx.x, c = threadIdx.x;
    v[c] = var[(size_t)h * kD + c];
    __syncthreads();
    const float mine = v[c];
    int rank = 0;
    for (int o = 0; o < kD; ++o) rank += (v[o] > mine) || (v[o] == mine && o < c);
    depth[(size_t)h * kD + c] = (uint8_t)(rank < n_channels ? kPlanes : 0);
}

}  // namespace

hipError_t launch_plan(const fathom_store &st, const float *q, int G, int B,
                       uint8_t *depth, hipStream_t s, uint32_t *zero) {
    hipLaunchKernelGGL(k_plan, dim3(st.n_heads), dim3(256), 0, s, q, st.var, G, B, depth, zero);
    return hipGetLastError();
}

hipError_t launch_plan_fixed(const fathom_store &st, int n_channels, uint8_t *depth,
                             hipStream_t s) {
    hipLaunchKernelGGL(k_plan_fixed, dim3(st.n_heads), dim3(kD), 0, s, st.var, n_channels,
                       depth);
    return hipGetLastError();
}

}  // namespace fathom
