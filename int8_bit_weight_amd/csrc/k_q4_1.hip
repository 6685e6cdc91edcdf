// k_q4_1.hip -- q4_1 kernels (placeholder until the q4_1 path lands).
#include "qmm_internal.h"

extern "C" {
size_t qmm_q4_1_packed_bytes(int64_t, int64_t) { return 0; }
qmm_status q4_1_repack(const void *, int64_t, int64_t, void *, size_t, void *) { return QMM_ERR_UNSUPPORTED; }
size_t qmm_q4_1_matmul_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }
qmm_status q4_1_matmul(const float *, int64_t, int64_t, int64_t, const void *, int64_t, float *, int64_t,
                       void *, size_t, void *) { return QMM_ERR_UNSUPPORTED; }
size_t qmm_q4_1_matmul_id_workspace_bytes(int64_t, int64_t, int64_t, int64_t, int64_t) { return 0; }
qmm_status q4_1_matmul_id(const float *, int64_t, int64_t, int64_t, const void *, int64_t, int64_t, size_t,
                          const int32_t *, int64_t, int64_t, float *, int64_t, int64_t, void *, size_t,
                          void *) { return QMM_ERR_UNSUPPORTED; }
}
