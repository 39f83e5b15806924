// Survival-ordered verify planner kernel: one 1024-thread workgroup, everything in LDS (the
// planner itself, and its sources, are in plan.h).
#include "plan.h"

namespace dspark {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanMax = 8192;   // B * gamma limit

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs p) {
  __shared__ plan::Smem<kPlanMax> sm;
  plan::run<kPlanThreads>(p, sm);
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  launch_kernel(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dspark
