// The backward's main kernel at head dims 16 and 32, in an object of its own.
//
// ffa_bwd.hip is built with the max-ILP machine scheduler, which schedules the
// D >= 64 kernels better but the D = 16 and 32 ones worse (same instructions, same
// results); this file takes the kernel template from there and instantiates the
// small head dims under the default scheduler.  ffa_bwd.hip declares these
// instances extern, so each is compiled once.
#define FFA_BWD_KERNELS_ONLY
#include "ffa_bwd.hip"

namespace ffa::bwd {

#define FFA_BWD_SMALL(D, T)                                                      \
  template __global__ void ffa_bwd_main<D, false, false, false, T>(BwdArgs);     \
  template __global__ void ffa_bwd_main<D, false, true, false, T>(BwdArgs);      \
  template __global__ void ffa_bwd_main<D, true, false, false, T>(BwdArgs);      \
  template __global__ void ffa_bwd_main<D, true, true, false, T>(BwdArgs);       \
  template __global__ void ffa_bwd_main<D, true, false, true, T>(BwdArgs);       \
  template __global__ void ffa_bwd_main<D, true, true, true, T>(BwdArgs);
FFA_BWD_SMALL(16, __bf16)
FFA_BWD_SMALL(16, _Float16)
FFA_BWD_SMALL(32, __bf16)
FFA_BWD_SMALL(32, _Float16)
#undef FFA_BWD_SMALL

}  // namespace ffa::bwd
