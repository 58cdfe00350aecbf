// decode.hip -- decode launcher: the 3-bit instantiation of the decode kernels
// (decode_impl.h) and the dispatch over the codecs (the other codecs are
// instantiated in decode_q2.hip and decode_q4.hip).
#include "decode_impl.h"

namespace moe {

template hipError_t launch_decode_t<kQ3G128>(const FwdArgs& f, const WsLayout& L, float* shared_out,
                                        int nsh, hipEvent_t join, hipStream_t s);
extern template hipError_t launch_decode_t<kQ4G32>(const FwdArgs& f, const WsLayout& L, float* shared_out,
                                        int nsh, hipEvent_t join, hipStream_t s);
extern template hipError_t launch_decode_t<kQ4G128>(const FwdArgs& f, const WsLayout& L, float* shared_out,
                                        int nsh, hipEvent_t join, hipStream_t s);
extern template hipError_t launch_decode_t<kQ2G128>(const FwdArgs& f, const WsLayout& L, float* shared_out,
                                        int nsh, hipEvent_t join, hipStream_t s);

hipError_t launch_decode(const FwdArgs& f, const WsLayout& L, float* shared_out, int nsh,
                         hipEvent_t join, hipStream_t s) {
  switch (codec_of(f.c->bits, f.c->group)) {
    case kQ3G128: return launch_decode_t<kQ3G128>(f, L, shared_out, nsh, join, s);
    case kQ4G32: return launch_decode_t<kQ4G32>(f, L, shared_out, nsh, join, s);
    case kQ2G128: return launch_decode_t<kQ2G128>(f, L, shared_out, nsh, join, s);
    case kQ4G128: return launch_decode_t<kQ4G128>(f, L, shared_out, nsh, join, s);
    default: return hipErrorInvalidValue;
  }
}

MOE_TRACE_EXPORT(decode)

}  // namespace moe
