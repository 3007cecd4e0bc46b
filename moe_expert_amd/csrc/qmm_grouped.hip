// placeholder until the grouped kernels land
#include "qmm_host.h"
extern "C" size_t qgemv_grouped_experts_workspace(int64_t, int, unsigned) { return 0; }
extern "C" int qgemv_grouped_experts(int, const void*, const void*, int64_t, int, const void*, int64_t, const uint8_t*,
                                     int64_t, int64_t, const void*, const int32_t*, const int32_t*, int, const int32_t*, int,
                                     float*, void*, size_t, unsigned, void*) { return QMM_EUNSUPPORTED; }
