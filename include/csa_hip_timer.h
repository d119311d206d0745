/*
 * csa_hip_timer.h — measurement support of libcsa_hip, not part of the
 * method's interface (include/csa_hip.h). Benchmarks use it to time one
 * kernel of the library's calls with HIP events recorded on the stream the
 * kernel is launched on.
 *
 * csa_kernel_timer_start() arms the timer for the next `max_launches`
 * launches of kernel `kernel_id` (a csa_kernel_id), made by any thread;
 * csa_kernel_timer_read() waits for the last recorded event, writes up to
 * `capacity` durations in milliseconds, returns how many launches were
 * recorded (negative on error) and disarms the timer. While the timer is
 * disarmed (the default) the library records nothing. The timer is guarded
 * by a lock, so concurrent calls are safe; launches of the armed kernel from
 * several threads are recorded in the order they take the lock. Not for use
 * under stream capture.
 */
#ifndef CSA_HIP_TIMER_H
#define CSA_HIP_TIMER_H

#include <stdint.h>

#include "csa_hip.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA_KID_COMPRESS = 1,
  CSA_KID_HCA_COMPRESS = 2,
  CSA_KID_QUANTIZE = 3,
  CSA_KID_INDEX_SCORE = 4,
  CSA_KID_TOPK = 5,
  CSA_KID_SPARSE_ATTN = 6,
  CSA_KID_DENSE_ATTN = 7,
  CSA_KID_ATTN_MERGE = 8,
  CSA_KID_ATTN_BWD = 9,
  CSA_KID_GEMM = 10
} csa_kernel_id;

csa_status csa_kernel_timer_start(int32_t kernel_id, int32_t max_launches);
int32_t csa_kernel_timer_read(float* ms_out, int32_t capacity);

#ifdef __cplusplus
}
#endif
#endif /* CSA_HIP_TIMER_H */
