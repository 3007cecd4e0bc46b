// qmm_host.h -- host-side helpers shared by the libqmm entry points (argument checks, launch
// status).  No device code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qmm.h"

namespace qmm {

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

inline int64_t row_bytes_of(int wtype, int64_t k) { return qmm_row_bytes(wtype, k); }

inline bool valid_wtype(int wtype) { return wtype == QMM_Q8_0 || wtype == QMM_IQ4_NL || wtype == QMM_CB3; }

// Status after a launch: QMM_EHIP if the runtime recorded a launch error.
inline int launch_status() {
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? QMM_OK : QMM_EHIP;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

constexpr int64_t kMaxK = 32768;

inline int64_t pow2_ceil(int64_t v) {
    int64_t p = 1;
    while (p < v) p <<= 1;
    return p;
}
constexpr uint64_t kMaxBufferBytes = 0xFFFFFFFFull;  // raw-buffer record range (32-bit offsets)
// Activation buffers: the kernels read zeros at their end (offset = size, plus up to 36 bytes),
// which must not wrap the 32-bit offset.
constexpr uint64_t kMaxActBytes = 0xFFFFFF00ull;

}  // namespace qmm
