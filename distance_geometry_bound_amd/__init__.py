"""distance_geometry_bound_amd: distance-bound triangle smoothing on MI355X.

The GPU work lives in the HIP library ``libdbs.so`` (C ABI declared in
``include/dbs.h``); this package is its thin Python binding.  The binding is
loaded lazily on first use so that the input generator (``gen``) can be
imported on machines without a GPU.
"""
__version__ = "0.1.0"

_API = ("smooth", "smooth_round", "smooth_rounds", "check", "lib", "DbsError", "auto_algo", "smooth_profiled", "PROF_KINDS", "smooth_range", "tightened",
        "bounds_from_restraints", "RESTRAINT_FLAGS", "pack", "unpack", "smooth_packed", "check_packed",
        "smooth_directed", "smooth_directed_range", "smooth_packed_directed", "lookahead_bands",
        "step_blocks", "schedule", "options", "Options", "AUTO",
        "ALGO_AUTO", "ALGO_PERK", "ALGO_LDS", "ALGO_BLOCKED", "CHECK_FLAGS",
        "INFEASIBLE_EARLY", "INFEASIBLE_END")


def __getattr__(name):
    if name in _API:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
