// C ABI entry points: validation, workspace sizing and dispatch (include/ffnwb.h).
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include "internal.hpp"

namespace ffnwb {

bool log_enabled() {
  static const bool on = [] {
    const char* v = getenv("FFNWB_LOG");
    return v != nullptr && v[0] != '\0' && v[0] != '0';
  }();
  return on;
}

void log_warn(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  fprintf(stderr, "[ffnwb] warning: ");
  vfprintf(stderr, fmt, ap);
  fprintf(stderr, "\n");
  va_end(ap);
}

// The caller's workspace: at least `need` bytes, and (when any is needed) non-NULL and
// 256-byte aligned, since the kernels store 16-byte vectors into the pieces carved from it.
static bool workspace_ok(const void* ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need) return false;
  return need == 0 || (ws != nullptr && reinterpret_cast<uintptr_t>(ws) % 256 == 0);
}

}  // namespace ffnwb

using namespace ffnwb;

extern "C" {

int ffnwb_abi_version(void) { return FFNWB_ABI_VERSION; }

size_t ffnwb_batching_desc_size(void) { return sizeof(ffnwb_batching_desc); }

size_t ffnwb_batching_ctx_desc_size(void) { return sizeof(ffnwb_batching_ctx_desc); }

size_t moe_unpermute_desc_size(void) { return sizeof(moe_unpermute_desc); }

size_t moe_permute_desc_size(void) { return sizeof(moe_permute_desc); }

size_t moe_update_expert_desc_size(void) { return sizeof(moe_update_expert_desc); }

const char* ffnwb_status_string(int status) {
  switch (status) {
    case FFNWB_OK: return "FFNWB_OK";
    case FFNWB_ERR_PARAM_NULLPTR: return "FFNWB_ERR_PARAM_NULLPTR: a required pointer is NULL";
    case FFNWB_ERR_PARAM_INVALID: return "FFNWB_ERR_PARAM_INVALID: a type, shape or range is not supported";
    case FFNWB_ERR_INNER_NULLPTR: return "FFNWB_ERR_INNER_NULLPTR: topK > 512 or unsupported probs shape";
    case FFNWB_ERR_WORKSPACE: return "FFNWB_ERR_WORKSPACE: workspace missing, smaller than required or not 256-byte aligned";
    case FFNWB_ERR_RUNTIME: return "FFNWB_ERR_RUNTIME: the HIP runtime rejected a launch";
    case FFNWB_ERR_SCRATCH:
      return "FFNWB_ERR_SCRATCH: the call needs more workspace than the no-allocation entry point holds";
    default: return "unknown ffnwb status";
  }
}

int ffnwb_batching_workspace_size(const ffnwb_batching_desc* d, size_t* ws_bytes) {
  if (ws_bytes == nullptr) return FFNWB_ERR_PARAM_NULLPTR;
  BatchingPlan p;
  const int st = plan_batching(d, &p);
  if (st != FFNWB_OK) return st;
  *ws_bytes = p.ws_bytes;
  return FFNWB_OK;
}

int ffnwb_batching(const ffnwb_batching_desc* d, void* workspace, size_t ws_bytes, void* stream) {
  BatchingPlan p;
  const int st = plan_batching(d, &p);
  if (st != FFNWB_OK) return st;
  if (!workspace_ok(workspace, ws_bytes, p.ws_bytes)) return FFNWB_ERR_WORKSPACE;
  return launch_batching(d, p, workspace, static_cast<hipStream_t>(stream));
}

int ffnwb_batching_ctx_workspace_size(const ffnwb_batching_ctx_desc* d, size_t* ws_bytes) {
  if (ws_bytes == nullptr) return FFNWB_ERR_PARAM_NULLPTR;
  BatchingCtxPlan p;
  const int st = plan_batching_ctx(d, &p);
  if (st != FFNWB_OK) return st;
  *ws_bytes = p.ws_bytes;
  return FFNWB_OK;
}

int ffnwb_batching_ctx(const ffnwb_batching_ctx_desc* d, void* workspace, size_t ws_bytes, void* stream) {
  BatchingCtxPlan p;
  const int st = plan_batching_ctx(d, &p);
  if (st != FFNWB_OK) return st;
  if (!workspace_ok(workspace, ws_bytes, p.ws_bytes)) return FFNWB_ERR_WORKSPACE;
  return launch_batching_ctx(d, p, workspace, static_cast<hipStream_t>(stream));
}

int moe_unpermute_workspace_size(const moe_unpermute_desc* d, size_t* ws_bytes) {
  if (ws_bytes == nullptr) return FFNWB_ERR_PARAM_NULLPTR;
  UnpermutePlan p;
  const int st = plan_unpermute(d, &p);
  if (st != FFNWB_OK) return st;
  *ws_bytes = p.ws_bytes;
  return FFNWB_OK;
}

int moe_unpermute(const moe_unpermute_desc* d, void* workspace, size_t ws_bytes, void* stream) {
  UnpermutePlan p;
  const int st = plan_unpermute(d, &p);
  if (st != FFNWB_OK) return st;
  if (!workspace_ok(workspace, ws_bytes, p.ws_bytes)) return FFNWB_ERR_WORKSPACE;
  return launch_unpermute(d, p, workspace, static_cast<hipStream_t>(stream));
}

int moe_permute_workspace_size(const moe_permute_desc* d, size_t* ws_bytes) {
  if (ws_bytes == nullptr) return FFNWB_ERR_PARAM_NULLPTR;
  PermutePlan p;
  const int st = plan_permute(d, &p);
  if (st != FFNWB_OK) return st;
  *ws_bytes = p.ws_bytes;
  return FFNWB_OK;
}

int moe_permute(const moe_permute_desc* d, void* workspace, size_t ws_bytes, void* stream) {
  PermutePlan p;
  const int st = plan_permute(d, &p);
  if (st != FFNWB_OK) return st;
  if (!workspace_ok(workspace, ws_bytes, p.ws_bytes)) return FFNWB_ERR_WORKSPACE;
  return launch_permute(d, p, workspace, static_cast<hipStream_t>(stream));
}

int moe_update_expert_workspace_size(const moe_update_expert_desc* d, size_t* ws_bytes) {
  if (ws_bytes == nullptr) return FFNWB_ERR_PARAM_NULLPTR;
  const int st = plan_update_expert(d);
  if (st != FFNWB_OK) return st;
  *ws_bytes = 0;
  return FFNWB_OK;
}

int moe_update_expert(const moe_update_expert_desc* d, void* workspace, size_t ws_bytes, void* stream) {
  (void)workspace;
  (void)ws_bytes;
  const int st = plan_update_expert(d);
  if (st != FFNWB_OK) return st;
  return launch_update_expert(d, static_cast<hipStream_t>(stream));
}

}  // extern "C"
