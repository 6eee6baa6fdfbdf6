// Upload of small int32 tables (block offsets, segment lists) into device
// memory, ordered on the caller's stream: the values ride in the kernel
// arguments of k_upload, so no host staging memory and no host wait is
// involved.  A table of n ints takes ceil(n / kUploadInts) launches.
#include "dbsa_device.hpp"

namespace dbsa {

__global__ __launch_bounds__(256) void k_upload(UploadArgs a) {
  const int32_t* v = kernarg_ints(offsetof(UploadArgs, v));
  for (int i = threadIdx.x; i < a.n; i += blockDim.x) a.dst[i] = v[i];
}

hipError_t launch_upload(const UploadArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(k_upload, dim3(1), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dbsa
