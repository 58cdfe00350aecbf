// decode_q4.hip -- the decode kernels (decode_impl.h) for 4-bit codes in groups
// of 32 and of 128.
#include "decode_impl.h"

namespace moe {
template hipError_t launch_decode_t<kQ4G32>(const FwdArgs& f, const WsLayout& L, float* shared_out,
                                        int nsh, hipEvent_t join, hipStream_t s);
template hipError_t launch_decode_t<kQ4G128>(const FwdArgs& f, const WsLayout& L, float* shared_out,
                                        int nsh, hipEvent_t join, hipStream_t s);
}  // namespace moe
