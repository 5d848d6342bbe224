/* C consumer check of include/coda.h: the header compiles as C99 (no C++ or HIP types in
 * the declarations), and every entry point it declares can be named from C. Compiled
 * (not run) by tests/test_c_abi.py. */
#include <stddef.h>

#include "coda.h"

typedef void (*any_fn)(void);

const any_fn coda_entry_points[] = {
    (any_fn)&coda_status_string,
    (any_fn)&coda_abi_version,
    (any_fn)&coda_build_source_hash,
    (any_fn)&coda_rowstat_num_partials,
    (any_fn)&coda_gemm_rmsnorm_fwd,
    (any_fn)&coda_gemm_rmsnorm_fwd_ws,
    (any_fn)&coda_gemm_rmsnorm_fwd_workspace_bytes,
    (any_fn)&coda_gemm_rmsnorm_fwd_noalloc,
    (any_fn)&coda_gemm_residual_rmsnorm_partials,
    (any_fn)&coda_gemm_rowscale,
    (any_fn)&coda_rowstat_reduce,
    (any_fn)&coda_rope_tables,
    (any_fn)&coda_gemm_rope,
    (any_fn)&coda_gemm_rope_ws,
    (any_fn)&coda_gemm_rope_persistent,
    (any_fn)&coda_gemm_swiglu,
    (any_fn)&coda_gemm_swiglu_ws,
    (any_fn)&coda_split_workspace_bytes,
    (any_fn)&coda_split_plan,
    (any_fn)&coda_gemm_rope_bwd,
    (any_fn)&coda_gemm_rope_bwd_ws,
    (any_fn)&coda_gemm_swiglu_bwd,
    (any_fn)&coda_gemm_swiglu_bwd_ws,
    (any_fn)&coda_gemm_rmsnorm_bwd_stats,
    (any_fn)&coda_gemm_rmsnorm_bwd_stats_ws,
    (any_fn)&coda_colstat_num_partials,
    (any_fn)&coda_rowdot_stat,
    (any_fn)&coda_colsum_reduce,
    (any_fn)&coda_gemm_rmsnorm_bwd_dx,
    (any_fn)&coda_gemm_rmsnorm_bwd_dx_ws,
    (any_fn)&coda_rmsnorm_bwd,
    (any_fn)&coda_gemm_cross_entropy,
    (any_fn)&coda_gemm_cross_entropy_ws,
    (any_fn)&coda_lse_reduce,
    (any_fn)&coda_baseline_gemm,
    (any_fn)&coda_baseline_residual_rmsnorm,
    (any_fn)&coda_baseline_rope,
    (any_fn)&coda_baseline_swiglu,
    (any_fn)&coda_baseline_rowdot,
    (any_fn)&coda_baseline_copy,
    (any_fn)&coda_baseline_mfma_loop,
    (any_fn)&coda_baseline_schedule_probe,
};
const size_t coda_entry_point_count = sizeof coda_entry_points / sizeof coda_entry_points[0];
