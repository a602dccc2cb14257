// Host-only declarations shared by the C ABI: the page size, the KV pool handle, error reporting and
// the configuration check.  No device code: the page allocator builds from this alone (also with host
// sanitizers).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "llmdec.h"

namespace llmdec {

constexpr int kPage = 16;  // tokens per KV page

llmdec_status set_error(llmdec_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
llmdec_status clear_error();
llmdec_status check_config(const llmdec_config *cfg, const char *who);

}  // namespace llmdec

// The opaque pool handle (host side).
struct llmdec_kv_pool {
  llmdec_config cfg;
  void *base;           // device base of the pool
  size_t bytes;
  int32_t num_pages;
  int32_t *stack;       // free-page stack; top = stack[top-1]
  int32_t top;
  uint8_t *is_free;     // per page: 1 if on the free list
};
