// sys_attn_mfma: RelayAttention's system-attention step on the matrix cores of gfx950
// for many stacked query rows (bf16 inputs, head_dim 128), as a launch of its own (the
// offline prefill's causal attention, and the system step alone); the decode step runs
// the same workgroups inside the streaming launch (stream_attn.hip).  The workgroup
// itself is in sys_attn_mfma.hpp.
#include "sys_attn_mfma.hpp"

namespace relay {

template <bool CAUSAL>
__global__ __launch_bounds__(mf::kThreads, 2) void sys_attn_mfma_kernel(SysArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  sys_mfma_workgroup<CAUSAL>(a, blockIdx.x, gridDim.x, lds_raw);
}

// The decode system step alone (non-causal): one workgroup of eight waves per CU.
__global__ __launch_bounds__(pp::kThreads, 1) void sys_attn_mfma_pp_kernel(SysArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  sys_pp_workgroup(a, blockIdx.x, gridDim.x, lds_raw);
}

hipError_t launch_sys_attn_pp(const SysArgs& a, int nwg, hipStream_t stream, const LaunchTiming* tm) {
  if (a.causal) return hipErrorInvalidValue;
  launch_kernel(sys_attn_mfma_pp_kernel, dim3(nwg), dim3(pp::kThreads), (uint32_t)kSysPPLds, stream, tm, a);
  return hipGetLastError();
}

hipError_t launch_sys_attn_mfma(const SysArgs& a, int nwg, hipStream_t stream, const LaunchTiming* tm) {
  if (a.causal)
    launch_kernel(sys_attn_mfma_kernel<true>, dim3(nwg), dim3(mf::kThreads), (uint32_t)kSysMfmaLds, stream, tm, a);
  else
    launch_kernel(sys_attn_mfma_kernel<false>, dim3(nwg), dim3(mf::kThreads), (uint32_t)kSysMfmaLds, stream, tm, a);
  return hipGetLastError();
}

}  // namespace relay
