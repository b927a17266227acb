// Host-side status handling and introspection of the C ABI.
#include <stdarg.h>
#include <stdio.h>

#include "common.h"

namespace {
thread_local char g_last_error[512] = "";
}

namespace csa_host {

csa_status fail(csa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_last_error[0] = '\0'; }

csa_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return CSA_OK;
}

bool fmt_valid_tensor(const csa_tensor* t, bool need_data) {
  if (t == nullptr || t->rows < 0 || t->dim <= 0) return false;
  if (need_data && t->rows > 0 && t->data == nullptr) return false;
  switch (t->fmt) {
    case CSA_F32:
    case CSA_BF16:
      return true;
    case CSA_FP8_MIXED:
      return t->dim == 512 && (t->rows == 0 || (t->scale != nullptr && t->rope != nullptr));
    case CSA_MXFP4:
      return t->dim % 32 == 0 && (t->rows == 0 || t->scale != nullptr);
    default:
      return false;
  }
}

int64_t rows_of(const csa_tensor* t) { return t == nullptr ? 0 : t->rows; }

csa_status batch_pages(const csa_batch* b, csa::BatchDev& d, const char* who) {
  d.pages = nullptr;
  d.page_stride = 0;
  d.page_shift = 0;
  if (b->kv_block_table == nullptr) return CSA_OK;
  const int32_t p = b->kv_block_rows;
  if (b->kv_block_stride < 1 || p < 1 || p > (1 << 20) || (p & (p - 1)) != 0)
    return fail(CSA_ERR_INVALID_ARGUMENT,
                "%s: kv_block_table needs kv_block_stride >= 1 and kv_block_rows a power of two in [1, 2^20]",
                who);
  d.pages = b->kv_block_table;
  d.page_stride = b->kv_block_stride;
  d.page_shift = __builtin_ctz((unsigned)p);
  return CSA_OK;
}

}  // namespace csa_host

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_status_string(csa_status s) {
  switch (s) {
    case CSA_OK: return "ok";
    case CSA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case CSA_ERR_UNSUPPORTED: return "unsupported";
    case CSA_ERR_WORKSPACE: return "workspace too small";
    case CSA_ERR_HIP: return "hip error";
    default: return "unknown status";
  }
}

const char* csa_last_error(void) { return g_last_error; }

}  // extern "C"
