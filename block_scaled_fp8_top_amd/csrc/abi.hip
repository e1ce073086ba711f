// Library-level entry points of libmoe_fp8: workspace sizes, status strings, version.
#include "common.h"

size_t moe_dispatch_workspace(int64_t T, int32_t k, int32_t E);
size_t moe_gemm_workspace(int64_t max_rows, int32_t groups);

extern "C" size_t moe_workspace_bytes(int op, int64_t rows_or_T, int32_t k, int32_t E, int32_t N, int32_t K) {
  (void)N;
  (void)K;
  if (rows_or_T < 0 || E < 1) return 0;
  switch (op) {
    case MOE_OP_DISPATCH:
      if (k < 1) return 0;
      return moe_dispatch_workspace(rows_or_T, k, E);
    case MOE_OP_GROUPED_GEMM:
      return moe_gemm_workspace(rows_or_T, E);
    default:
      return 0;
  }
}

extern "C" const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or not a required multiple";
    case MOE_ERR_DTYPE: return "unsupported dtype";
    case MOE_ERR_ARG: return "invalid argument or router configuration";
    case MOE_ERR_HIP: return "HIP runtime error at launch";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

extern "C" const char* moe_version(void) { return "moe_fp8 0.1 gfx950"; }
