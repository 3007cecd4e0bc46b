// placeholder until the prefill kernels land
#include "qmm_host.h"
extern "C" size_t qgemm_prefill_experts_workspace(int, int64_t, int64_t, unsigned) { return 0; }
extern "C" int qgemm_prefill_experts(int, const void*, const void*, int64_t, int, const void*, int64_t, int, int64_t,
                                     int64_t, const uint16_t*, int64_t, const int32_t*, const int32_t*, int64_t, float*,
                                     void*, size_t, unsigned, void*) { return QMM_EUNSUPPORTED; }
