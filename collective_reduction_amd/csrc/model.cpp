// α-β cost model of the pages' collectives (declared in ccl_sim.h).  Host
// arithmetic only; it prices the algorithms on a network for context and
// never touches the GPU.
//
// Pages cited:
//   [PRIMS] "通信与互联（01）：集合通信原语与代价模型——α-β 模型与 ring all-reduce"
//           §四 (α-β model), §五 (ring), §六 (tree), §七 (algbw / busbw),
//           §八 (two-level)

#include <cmath>

#include "ccl_sim.h"

namespace {

bool valid_model_coll(int c) { return c >= CCL_SIM_MODEL_ALLREDUCE && c <= CCL_SIM_MODEL_REDUCE; }

struct Phase {
  double steps;
  double bytes;  // per rank
};

// Ring schedule of one collective: how many steps and how many bytes each
// rank moves over its one outgoing link ([PRIMS] §五).
Phase ring_phase(int coll, int n, double s) {
  const double frac = double(n - 1) / double(n);
  switch (coll) {
    case CCL_SIM_MODEL_ALLREDUCE: return {2.0 * (n - 1), 2.0 * frac * s};
    case CCL_SIM_MODEL_ALL_GATHER:
    case CCL_SIM_MODEL_REDUCE_SCATTER:
    case CCL_SIM_MODEL_ALL_TO_ALL: return {double(n - 1), frac * s};
    default: return {double(n - 1), s};  // broadcast / reduce: a pipelined chain
  }
}

}  // namespace

extern "C" {

double ccl_sim_busbw_factor(ccl_sim_model_coll_t coll, int nranks) {
  if (!valid_model_coll(coll) || nranks < 1) return -1.0;
  const double frac = double(nranks - 1) / double(nranks);
  if (coll == CCL_SIM_MODEL_ALLREDUCE) return 2.0 * frac;
  if (coll == CCL_SIM_MODEL_BROADCAST || coll == CCL_SIM_MODEL_REDUCE) return 1.0;
  return frac;
}

ccl_sim_result_t ccl_sim_model_estimate(ccl_sim_model_coll_t coll, ccl_sim_model_algo_t algo, int nranks,
                                        double size_bytes, const ccl_sim_link_params_t* link,
                                        ccl_sim_model_estimate_t* out) {
  if (!valid_model_coll(coll) || nranks < 1 || !(size_bytes >= 0.0) || link == nullptr || out == nullptr ||
      !(link->alpha_s >= 0.0) || !(link->beta_bytes_per_s > 0.0))
    return CCL_SIM_INVALID_ARGUMENT;
  double lat = 0.0, bw = 0.0, steps = 0.0;
  if (algo == CCL_SIM_ALGO_RING) {
    const Phase p = ring_phase(coll, nranks, size_bytes);
    steps = p.steps;
    lat = p.steps * link->alpha_s;
    bw = p.bytes / link->beta_bytes_per_s;
  } else if (algo == CCL_SIM_ALGO_DOUBLE_TREE) {
    if (coll != CCL_SIM_MODEL_ALLREDUCE) return CCL_SIM_UNSUPPORTED;
    // up the tree and back down: 2·ceil(log2 N) steps; two trees of S/2
    // each put 2S through every rank ([PRIMS] §六)
    steps = nranks > 1 ? 2.0 * std::ceil(std::log2(double(nranks))) : 0.0;
    lat = steps * link->alpha_s;
    bw = nranks > 1 ? 2.0 * size_bytes / link->beta_bytes_per_s : 0.0;
  } else if (algo == CCL_SIM_ALGO_TWO_LEVEL) {
    if (coll != CCL_SIM_MODEL_ALLREDUCE) return CCL_SIM_UNSUPPORTED;
    const int ppn = link->ranks_per_node;
    if (ppn < 1 || nranks % ppn != 0 || !(link->alpha_intra_s >= 0.0) || !(link->beta_intra_bytes_per_s > 0.0))
      return CCL_SIM_INVALID_ARGUMENT;
    // intra ReduceScatter, inter AllReduce on one shard, intra AllGather (the
    // AllGather costs what the ReduceScatter costs) ([PRIMS] §八)
    const Phase intra = ring_phase(CCL_SIM_MODEL_REDUCE_SCATTER, ppn, size_bytes);
    const Phase inter = ring_phase(CCL_SIM_MODEL_ALLREDUCE, nranks / ppn, size_bytes / ppn);
    steps = 2.0 * intra.steps + inter.steps;
    lat = 2.0 * intra.steps * link->alpha_intra_s + inter.steps * link->alpha_s;
    bw = 2.0 * intra.bytes / link->beta_intra_bytes_per_s + inter.bytes / link->beta_bytes_per_s;
  } else {
    return CCL_SIM_INVALID_ARGUMENT;
  }
  const double t = lat + bw;
  out->time_s = t;
  out->latency_s = lat;
  out->bandwidth_s = bw;
  out->steps = steps;
  out->latency_fraction = t > 0.0 ? lat / t : 0.0;
  out->algbw_gbps = t > 0.0 ? size_bytes / t / 1e9 : 0.0;
  out->busbw_gbps = out->algbw_gbps * ccl_sim_busbw_factor(coll, nranks);
  return CCL_SIM_SUCCESS;
}

}  // extern "C"
