// Dispatch between the shape-specialised routing kernels and the generic one.
#include <hip/hip_runtime.h>

#include "route_common.cuh"
#include "route_internal.h"

namespace moe_route {

route_status_t launch_route_generic(const RouteProblem& p);

route_status_t launch_route(const RouteProblem& p) { return launch_route_generic(p); }

}  // namespace moe_route
