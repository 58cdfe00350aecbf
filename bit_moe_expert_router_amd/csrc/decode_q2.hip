// decode_q2.hip -- the decode kernels (decode_impl.h) for 2-bit codes in groups
// of 128.
#include "decode_impl.h"

namespace moe {
template hipError_t launch_decode_t<kQ2G128>(const FwdArgs& f, const WsLayout& L, float* shared_out,
                                        int nsh, hipEvent_t join, hipStream_t s);
}  // namespace moe
