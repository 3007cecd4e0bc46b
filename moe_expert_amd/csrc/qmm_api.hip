// qmm_api.hip -- format sizes, version and status strings of libqmm (host only).
#include "qmm_host.h"

extern "C" int qmm_version(void) { return 100; }

extern "C" const char* qmm_status_str(int status) {
    switch (status) {
        case QMM_OK: return "ok";
        case QMM_EINVAL: return "invalid argument";
        case QMM_EUNSUPPORTED: return "unsupported shape or format (declined)";
        case QMM_EALIGN: return "misaligned pointer or stride";
        case QMM_EHIP: return "HIP launch error";
        case QMM_ESPACE: return "workspace too small";
        default: return "unknown status";
    }
}

extern "C" int64_t qmm_row_bytes(int wtype, int64_t k) {
    if (k <= 0) return 0;
    switch (wtype) {
        case QMM_Q8_0: return k % 32 ? 0 : (k / 32) * 34;
        case QMM_IQ4_NL: return k % 32 ? 0 : (k / 32) * 18;
        case QMM_CB3: return k % 256 ? 0 : (k / 256) * 110;
        case QMM_F16: return 2 * k;
        default: return 0;
    }
}
