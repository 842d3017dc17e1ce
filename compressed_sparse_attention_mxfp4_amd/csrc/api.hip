// C ABI entry points that are not tied to one kernel family.
#include "common.h"
#include "index_common.h"

extern "C" size_t csa2_index_ws_bytes(int op, int32_t B, int32_t T, int32_t max_n,
                                      int32_t pool_blocks);
extern "C" size_t csa2_attn_ws_bytes(int32_t B, int32_t T, int32_t H, int32_t topk);

extern "C" size_t csa2_workspace_bytes(int op, int32_t B, int32_t T, int32_t heads,
                                       int32_t max_n_entries, int32_t topk) {
  if (B <= 0 || T <= 0 || heads <= 0) return 0;
  switch (op) {
    case CSA2_OP_INDEX_FULL:
      if (max_n_entries <= 0) return 0;
      return csa2_index_ws_bytes(op, B, T, max_n_entries, CSA2_MAX_POOL_BLOCKS);
    case CSA2_OP_INDEX_REINDEX:
      return csa2_index_ws_bytes(op, B, T, 0, CSA2_MAX_POOL_BLOCKS);
    case CSA2_OP_SPARSE_ATTN:
      if (topk <= 0) return 0;
      return csa2_attn_ws_bytes(B, T, heads, topk);
    default:
      return 0;
  }
}

extern "C" const char* csa2_status_str(int status) {
  switch (status) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_INVALID_ARG: return "invalid argument";
    case CSA2_ERR_UNSUPPORTED: return "unsupported size or shape";
    case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA2_ERR_LAUNCH: return "kernel launch failed";
    case CSA2_ERR_SCRATCH: return "request exceeds the fixed scratch of the no-allocation call";
    default: return "unknown status";
  }
}

extern "C" int csa2_abi_version(void) { return 108; }

namespace csa2 {
KernelEvents& kernel_events(int kernel) {
  static KernelEvents table[CSA2_K_COUNT];
  return table[(kernel > 0 && kernel < CSA2_K_COUNT) ? kernel : 0];
}
}  // namespace csa2

extern "C" int csa2_time_kernel(int kernel, void* start_event, void* stop_event) {
  if (kernel <= 0 || kernel >= CSA2_K_COUNT) return CSA2_ERR_INVALID_ARG;
  if ((start_event == nullptr) != (stop_event == nullptr)) return CSA2_ERR_INVALID_ARG;
  csa2::KernelEvents& e = csa2::kernel_events(kernel);
  e.start = reinterpret_cast<hipEvent_t>(start_event);
  e.stop = reinterpret_cast<hipEvent_t>(stop_event);
  return CSA2_OK;
}

extern "C" int csa2_test_select_path(int mode) {
  if (mode < 0 || mode > 2) return CSA2_ERR_INVALID_ARG;
  csa2::select_mode() = mode;
  return CSA2_OK;
}
