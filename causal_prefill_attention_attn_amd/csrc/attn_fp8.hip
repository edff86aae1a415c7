#include <hip/hip_runtime.h>
#include "attn_kernels.h"
namespace cpattn {
int launch_attn_fp8(const void*, const void*, const void*, void*, float*, int, int, int, int, float,
                    int, float, float, float, hipStream_t) {
  return -1;
}
}  // namespace cpattn
