// Error reporting and the configuration check of the C ABI (host code only).
#include <stdarg.h>
#include <stdio.h>

#include "host.h"

namespace llmdec {

static thread_local char g_err[512] = "";

llmdec_status set_error(llmdec_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

llmdec_status clear_error() {
  g_err[0] = 0;
  return LLMDEC_OK;
}

llmdec_status check_config(const llmdec_config *c, const char *who) {
  if (!c) return set_error(LLMDEC_E_INVALID, "%s: config is NULL", who);
  if (c->n_layers <= 0 || c->hidden <= 0 || c->n_heads <= 0 || c->head_dim <= 0 || c->intermediate <= 0 ||
      c->vocab <= 0)
    return set_error(LLMDEC_E_INVALID, "%s: config sizes must be positive", who);
  if (c->page_size != kPage)
    return set_error(LLMDEC_E_UNSUPPORTED, "%s: page_size must be %d, got %d", who, kPage, c->page_size);
  if (c->head_dim != 64 && c->head_dim != 128)
    return set_error(LLMDEC_E_UNSUPPORTED, "%s: head_dim must be 64 or 128, got %d", who, c->head_dim);
  if (c->n_heads * c->head_dim != c->hidden)
    return set_error(LLMDEC_E_INVALID, "%s: hidden (%d) != n_heads (%d) * head_dim (%d)", who, c->hidden, c->n_heads,
                     c->head_dim);
  if (c->n_kv_heads <= 0 || c->n_heads % c->n_kv_heads)
    return set_error(LLMDEC_E_INVALID, "%s: n_kv_heads (%d) must divide n_heads (%d)", who, c->n_kv_heads,
                     c->n_heads);
  if (c->hidden % 32 || c->intermediate % 16 || c->vocab % 16)
    return set_error(LLMDEC_E_INVALID, "%s: hidden must be a multiple of 32, intermediate and vocab of 16", who);
  if (c->hidden > 8192 || c->intermediate > 16384)
    return set_error(LLMDEC_E_UNSUPPORTED, "%s: hidden <= 8192 and intermediate <= 16384 are supported", who);
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f))
    return set_error(LLMDEC_E_INVALID, "%s: rms_eps must be >= 0 and rope_theta > 0", who);
  return LLMDEC_OK;
}

}  // namespace llmdec

extern "C" const char *llmdec_last_error(void) { return llmdec::g_err; }
