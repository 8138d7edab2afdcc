// kvq_vq.hip -- product-VQ encode/decode (in progress).
#include "kvq_internal.h"
namespace kvq {
hipError_t launch_vq_encode(const VqArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_vq_decode(const VqArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace kvq
