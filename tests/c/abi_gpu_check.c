/*
 * The C ABI end to end from plain C11 on a GPU, without Python or torch:
 * device buffers from hipMalloc, the pointer arrays on the host stack, the
 * worked example of four ranks by twenty int64 elements (x^(r)_i = 100 r + i,
 * every rank's result 600 + 4 i, shard r = elements 5r .. 5r + 4 of it),
 * through ReduceScatter then AllGather and through AllReduce, for every
 * schedule, each call on its own workspace sized by ccl_sim_workspace_size.
 * Prints "ok" and returns 0 when every value matches; otherwise names the
 * failing check and returns 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>

#include "ccl_sim.h"

#define N 4
#define M 20
#define Q 5

static int failures = 0;

#define CHECK(cond)                                        \
  do {                                                     \
    if (!(cond)) {                                         \
      printf("FAILED line %d: %s\n", __LINE__, #cond);     \
      ++failures;                                          \
    }                                                      \
  } while (0)

static void* device_alloc(size_t bytes) {
  void* p = NULL;
  if (bytes && hipMalloc(&p, bytes) != hipSuccess) {
    printf("hipMalloc of %zu bytes failed\n", bytes);
    return NULL;
  }
  return p;
}

int main(void) {
  int64_t host[N][M];
  for (int r = 0; r < N; ++r)
    for (int i = 0; i < M; ++i) host[r][i] = 100 * r + i;

  void* send[N];
  void* full[N];
  void* shard[N];
  for (int r = 0; r < N; ++r) {
    send[r] = device_alloc(M * sizeof(int64_t));
    full[r] = device_alloc(M * sizeof(int64_t));
    shard[r] = device_alloc(Q * sizeof(int64_t));
    if (!send[r] || !full[r] || !shard[r]) return 1;
    CHECK(hipMemcpy(send[r], host[r], M * sizeof(int64_t), hipMemcpyHostToDevice) == hipSuccess);
  }

  const ccl_sim_schedule_t schedules[] = {CCL_SIM_DIRECT, CCL_SIM_RING_STEPWISE, CCL_SIM_RING_PERSISTENT,
                                          CCL_SIM_RECURSIVE, CCL_SIM_RING_CHAINED, CCL_SIM_RECURSIVE_CHAINED};
  for (unsigned k = 0; k < sizeof(schedules) / sizeof(schedules[0]); ++k) {
    const ccl_sim_schedule_t s = schedules[k];
    const size_t ws_bytes = ccl_sim_workspace_size(CCL_SIM_COLL_ALLREDUCE, N, M, CCL_SIM_INT64, s);
    const size_t ws_rs = ccl_sim_workspace_size(CCL_SIM_COLL_REDUCE_SCATTER, N, M, CCL_SIM_INT64, s);
    const size_t ws_ag = ccl_sim_workspace_size(CCL_SIM_COLL_ALL_GATHER, N, M, CCL_SIM_INT64, s);
    size_t need = ws_bytes > ws_rs ? ws_bytes : ws_rs;
    need = need > ws_ag ? need : ws_ag;
    void* ws = device_alloc(need);
    if (need && !ws) return 1;

    int64_t got[M];
    if (s == CCL_SIM_RING_PERSISTENT) {
      /* ROCm can refuse a cooperative launch while another process on the
       * GPU holds cooperative launch resources; the call then says so */
      const ccl_sim_result_t rc = ccl_sim_allreduce((const void* const*)send, full, N, M, CCL_SIM_INT64, CCL_SIM_SUM, s,
                                                    ws, need, NULL);
      CHECK(rc == CCL_SIM_SUCCESS || rc == CCL_SIM_UNSUPPORTED);
      CHECK(hipDeviceSynchronize() == hipSuccess);
      if (rc == CCL_SIM_UNSUPPORTED) {
        printf("persistent ring refused here: %s\n", ccl_sim_last_error());
        if (ws) hipFree(ws);
        continue;
      }
    }
    CHECK(ccl_sim_reduce_scatter((const void* const*)send, shard, N, M, Q, CCL_SIM_INT64, CCL_SIM_SUM, s, ws, need,
                                 NULL) == CCL_SIM_SUCCESS);
    CHECK(ccl_sim_all_gather((const void* const*)shard, full, N, Q, M, CCL_SIM_INT64, s, ws, need, NULL) ==
          CCL_SIM_SUCCESS);
    CHECK(hipDeviceSynchronize() == hipSuccess);
    for (int r = 0; r < N; ++r) {
      int64_t sh[Q];
      CHECK(hipMemcpy(sh, shard[r], sizeof(sh), hipMemcpyDeviceToHost) == hipSuccess);
      for (int j = 0; j < Q; ++j) CHECK(sh[j] == 600 + 4 * (Q * r + j));
      CHECK(hipMemcpy(got, full[r], sizeof(got), hipMemcpyDeviceToHost) == hipSuccess);
      for (int i = 0; i < M; ++i) CHECK(got[i] == 600 + 4 * i);
    }

    for (int r = 0; r < N; ++r) CHECK(hipMemset(full[r], 0, M * sizeof(int64_t)) == hipSuccess);
    CHECK(ccl_sim_allreduce((const void* const*)send, full, N, M, CCL_SIM_INT64, CCL_SIM_SUM, s, ws, need, NULL) ==
          CCL_SIM_SUCCESS);
    CHECK(hipDeviceSynchronize() == hipSuccess);
    for (int r = 0; r < N; ++r) {
      CHECK(hipMemcpy(got, full[r], sizeof(got), hipMemcpyDeviceToHost) == hipSuccess);
      for (int i = 0; i < M; ++i) CHECK(got[i] == 600 + 4 * i);
    }
    if (s == CCL_SIM_RING_PERSISTENT) {
      int aborted = -1;
      CHECK(ccl_sim_persistent_aborted(ws, &aborted) == CCL_SIM_SUCCESS && aborted == 0);
    }
    if (ws) CHECK(hipFree(ws) == hipSuccess);
    if (failures) printf("schedule %d failed\n", (int)s);
  }

  /* a rejected call leaves the outputs untouched */
  for (int r = 0; r < N; ++r) CHECK(hipMemset(shard[r], 0, Q * sizeof(int64_t)) == hipSuccess);
  CHECK(ccl_sim_reduce_scatter((const void* const*)send, shard, N, M - 1, Q, CCL_SIM_INT64, CCL_SIM_SUM,
                               CCL_SIM_DIRECT, NULL, 0, NULL) == CCL_SIM_CAPACITY_MISMATCH);
  CHECK(hipDeviceSynchronize() == hipSuccess);
  for (int r = 0; r < N; ++r) {
    int64_t sh[Q];
    CHECK(hipMemcpy(sh, shard[r], sizeof(sh), hipMemcpyDeviceToHost) == hipSuccess);
    for (int j = 0; j < Q; ++j) CHECK(sh[j] == 0);
  }

  for (int r = 0; r < N; ++r) {
    hipFree(send[r]);
    hipFree(full[r]);
    hipFree(shard[r]);
  }
  if (failures == 0) printf("ok\n");
  return failures == 0 ? 0 : 1;
}
