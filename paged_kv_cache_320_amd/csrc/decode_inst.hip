// Decode kernels for one (key/value format, query/output format, head_dim), chosen at
// compile time with -DPA_INST_KT=<format> -DPA_INST_QT=<format> -DPA_INST_D=<64|128>.
// build.py compiles this file once per supported combination (in parallel); decode.hip
// picks the instance.
#include "decode_kernels.hpp"

#if !defined(PA_INST_KT) || !defined(PA_INST_QT) || !defined(PA_INST_D)
#error "define PA_INST_KT, PA_INST_QT and PA_INST_D"
#endif

#define PA_CAT6(a, b, c, d, e, f) a##b##c##d##e##f
#define PA_NAME(kt, qt, d) PA_CAT6(decode_launch_, kt, _, qt, _d, d)

namespace pagedkv {

bool PA_NAME(PA_INST_KT, PA_INST_QT, PA_INST_D)(int B, int GS, const decode_impl::Launch& a) {
  return decode_impl::dispatch_b<PA_INST_KT, PA_INST_QT, PA_INST_D>(B, GS, a);
}

}  // namespace pagedkv
