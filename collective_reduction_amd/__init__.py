"""ReduceScatter + AllGather AllReduce over N virtual ranks on one MI355X.

The compute path is the C-ABI library ``libccl_sim.so`` (hand-written HIP
for gfx950, declared in ``include/ccl_sim.h``); ``collective_reduction_amd.
ccl_sim`` is its thin ctypes binding with the same function names.  The
binding is loaded on first use of any of its names, so importing the
package (or its ``inputs`` module) does not touch the GPU; using a binding
name when the library has not been built raises at once — there is no CPU
fallback.
"""

_BINDING_NAMES = (
    "ccl_sim_reduce_scatter",
    "ccl_sim_all_gather",
    "ccl_sim_allreduce",
    "ccl_sim_pad_identity",
    "ccl_sim_workspace_size",
    "ccl_sim_algorithmic_bytes",
    "ccl_sim_ring_owner",
    "ccl_sim_ring_route",
    "ccl_sim_launch_count",
    "ccl_sim_result_string",
    "ccl_sim_version",
    "ccl_sim_model_estimate",
    "ccl_sim_busbw_factor",
    "ccl_sim_recursive_route",
    "Workspace",
    "CclSimError",
)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import ccl_sim

        return getattr(ccl_sim, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")


__all__ = list(_BINDING_NAMES)
