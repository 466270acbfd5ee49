// Helpers shared by the C-ABI sources: the per-thread error text, argument checks, workspace
// rounding, and dispatch of a GEMM to the bf16 or fp32 kernel family.
#pragma once
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <string>

#include "common.h"
#include "zdit.h"

namespace zdit {

// text behind zdit_last_error() on the calling thread
std::string& api_error_text();

inline zdit_status fail(zdit_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  api_error_text() = buf;
  return code;
}

inline zdit_status ok() {
  api_error_text().clear();
  return ZDIT_OK;
}

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess) return fail(ZDIT_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t al256(size_t n) { return (n + 255) & ~(size_t)255; }
inline int act_bytes(int precision) { return precision == ZDIT_BF16 ? 2 : 4; }
inline int round_up(int v, int m) { return (v + m - 1) / m * m; }

// every row written, rows of one "branch" of M rows at ld elements apart
inline RowMap compact_rows(int M, int64_t ld) {
  RowMap r;
  r.rows_per_batch = M > 0 ? M : 1;
  r.batch_stride = 0;
  r.ld = ld;
  for (int i = 0; i < kMaxBatch; ++i) r.valid[i] = M;
  return r;
}

inline hipError_t gemm(int precision, int epi, const GemmArgs& g, hipStream_t s) {
  return precision == ZDIT_BF16 ? launch_gemm_bf16(epi, g, s) : launch_gemm_f32(epi, g, s);
}

}  // namespace zdit
