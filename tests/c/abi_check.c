/*
 * The C ABI used from plain C11: include/ccl_sim.h compiles as C, and the
 * planning, model and validation entry points behave as the header states.
 * Nothing here needs a GPU: every call below either plans on the host or is
 * rejected by validation before any HIP call.  Prints "ok" and returns 0
 * when every check holds; otherwise names the failed check and returns 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ccl_sim.h"

static int failures = 0;

#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      printf("FAILED line %d: %s\n", __LINE__, #cond);           \
      ++failures;                                                \
    }                                                            \
  } while (0)

int main(void) {
  CHECK(ccl_sim_version() == CCL_SIM_VERSION);

  /* workspace sizes: none for the direct schedule with N <= 64; the ring's
   * double-buffered partials 2·N·q·4 at N = 8, M = 2^20 float32 */
  CHECK(ccl_sim_workspace_size(CCL_SIM_COLL_ALLREDUCE, 8, 1u << 20, CCL_SIM_FLOAT32, CCL_SIM_DIRECT) == 0);
  CHECK(ccl_sim_workspace_size(CCL_SIM_COLL_ALLREDUCE, 8, 1u << 20, CCL_SIM_FLOAT32, CCL_SIM_RING_STEPWISE) ==
        (size_t)2 * 8 * (1u << 17) * 4);
  CHECK(ccl_sim_workspace_size(CCL_SIM_COLL_ALLREDUCE, 8, 1u << 20, CCL_SIM_FLOAT32, CCL_SIM_RING_CHAINED) ==
        (size_t)8 * (1u << 17) * 4);
  CHECK(ccl_sim_workspace_size(CCL_SIM_COLL_ALLREDUCE, 0, 100, CCL_SIM_FLOAT32, CCL_SIM_DIRECT) == (size_t)-1);

  /* algorithmic bytes of the bench step, N = 8, M = 2^28 float32 */
  const uint64_t m = (uint64_t)1 << 28;
  CHECK(ccl_sim_algorithmic_bytes(CCL_SIM_COLL_REDUCE_SCATTER, 8, m, CCL_SIM_FLOAT32, CCL_SIM_DIRECT) == 9 * m * 4);
  CHECK(ccl_sim_algorithmic_bytes(CCL_SIM_COLL_ALLREDUCE, 8, m, CCL_SIM_FLOAT32, CCL_SIM_RING_STEPWISE) ==
        5 * 7 * m * 4);

  /* launch counts: 2(N-1) ring steps, one persistent or chained launch, 2·log2 N recursive steps */
  CHECK(ccl_sim_launch_count(CCL_SIM_COLL_ALLREDUCE, 256, 1000, CCL_SIM_RING_STEPWISE, 0) == 510);
  CHECK(ccl_sim_launch_count(CCL_SIM_COLL_ALLREDUCE, 256, 1000, CCL_SIM_RING_PERSISTENT, 0) == 1);
  CHECK(ccl_sim_launch_count(CCL_SIM_COLL_ALLREDUCE, 256, 1000, CCL_SIM_RING_CHAINED, 0) == 1);
  CHECK(ccl_sim_launch_count(CCL_SIM_COLL_ALLREDUCE, 256, 1000, CCL_SIM_RECURSIVE, 0) == 16);
  CHECK(ccl_sim_launch_count(CCL_SIM_COLL_ALLREDUCE, 256, 1000, CCL_SIM_RECURSIVE_CHAINED, 0) == 1);

  /* ring routing of [RING] §2 at N = 4: step 0, rank 0 sends chunk 0 and receives chunk 3 */
  int send_chunk = -1, recv_chunk = -1;
  CHECK(ccl_sim_ring_route(4, 0, 0, 0, &send_chunk, &recv_chunk) == CCL_SIM_SUCCESS);
  CHECK(send_chunk == 0 && recv_chunk == 3);
  CHECK(ccl_sim_ring_owner(4, 3) == 0);

  /* recursive halving at N = 8, step 1: rank 1 pairs with rank 5 */
  int partner = -1;
  size_t first = 0, nblocks = 0;
  CHECK(ccl_sim_recursive_route(8, 0, 1, 1, &partner, &first, &nblocks) == CCL_SIM_SUCCESS);
  CHECK(partner == 5);

  /* the alpha-beta model: [PRIMS]'s printed run of 8 ranks, 64 KiB, alpha 10 us, beta 25 GB/s -> 144.6 us */
  ccl_sim_link_params_t link;
  memset(&link, 0, sizeof link);
  link.alpha_s = 10e-6;
  link.beta_bytes_per_s = 25e9;
  ccl_sim_model_estimate_t est;
  CHECK(ccl_sim_model_estimate(CCL_SIM_MODEL_ALLREDUCE, CCL_SIM_ALGO_RING, 8, 65536.0, &link, &est) ==
        CCL_SIM_SUCCESS);
  CHECK(fabs(est.time_s * 1e6 - 144.6) < 0.05);
  CHECK(fabs(ccl_sim_busbw_factor(CCL_SIM_MODEL_ALLREDUCE, 8) - 1.75) < 1e-12);

  /* validation before any HIP call: the capacity mismatch of a
   * ReduceScatter whose sendcount is not nranks·recvcount */
  static float a[8][16], b[8][2];
  const void* sends[8];
  void* recvs[8];
  for (int r = 0; r < 8; ++r) {
    sends[r] = a[r];
    recvs[r] = b[r];
  }
  CHECK(ccl_sim_reduce_scatter(sends, recvs, 8, 15, 2, CCL_SIM_FLOAT32, CCL_SIM_SUM, CCL_SIM_DIRECT, NULL, 0, NULL) ==
        CCL_SIM_CAPACITY_MISMATCH);
  CHECK(strlen(ccl_sim_last_error()) > 0);
  CHECK(ccl_sim_allreduce(sends, recvs, 8, 16, CCL_SIM_FLOAT32, CCL_SIM_SUM, (ccl_sim_schedule_t)9, NULL, 0, NULL) ==
        CCL_SIM_INVALID_ARGUMENT);
  CHECK(ccl_sim_allreduce(sends, recvs, 6, 16, CCL_SIM_FLOAT32, CCL_SIM_SUM, CCL_SIM_RECURSIVE, NULL, 0, NULL) ==
        CCL_SIM_UNSUPPORTED);
  CHECK(strcmp(ccl_sim_result_string(CCL_SIM_SUCCESS), "") != 0);
  /* the watchdog query validates its pointers before any HIP call */
  int aborted = -1;
  CHECK(ccl_sim_persistent_aborted(NULL, &aborted) == CCL_SIM_INVALID_ARGUMENT && aborted == -1);
  CHECK(ccl_sim_persistent_aborted(sends[0], NULL) == CCL_SIM_INVALID_ARGUMENT);
  /* the persistent ring's step ordering, with CCL_SIM_PERSISTENT_SYNC unset:
     step flags for steps (N chunks of ceil(M/N)) of up to 2^26 elements */
  CHECK(ccl_sim_persistent_ordering(CCL_SIM_COLL_ALLREDUCE, 256, 1u << 22) == CCL_SIM_ORDER_FLAGS);
  CHECK(ccl_sim_persistent_ordering(CCL_SIM_COLL_ALLREDUCE, 8, (size_t)1 << 28) == CCL_SIM_ORDER_GRID);
  CHECK(ccl_sim_persistent_ordering(CCL_SIM_COLL_ALLREDUCE, 8, (size_t)1 << 26) == CCL_SIM_ORDER_FLAGS);
  CHECK(ccl_sim_persistent_ordering(CCL_SIM_COLL_ALLREDUCE, 1, 1000) == 0);
  CHECK(ccl_sim_persistent_ordering((ccl_sim_coll_t)7, 8, 1000) == -1);

  if (failures == 0) printf("ok\n");
  return failures == 0 ? 0 : 1;
}
