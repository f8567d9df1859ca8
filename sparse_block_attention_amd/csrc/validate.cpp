// Host-only argument checks and status reporting of the C ABI (no HIP calls).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "apb_host.h"

namespace apb_host {

static thread_local char g_err[512];

apb_status fail(apb_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_err[0] = '\0'; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

apb_status check_problem(const apb_problem *pr) {
  if (pr == nullptr) return fail(APB_ERR_INVALID_ARGUMENT, "problem is NULL");
  const int Hq = pr->n_q_heads, Hkv = pr->n_kv_heads;
  if (Hkv < 1) return fail(APB_ERR_INVALID_ARGUMENT, "n_kv_heads = %d, need >= 1", Hkv);
  if (Hq < 1 || Hq % Hkv != 0)
    return fail(APB_ERR_INVALID_ARGUMENT, "n_q_heads = %d is not a positive multiple of n_kv_heads = %d", Hq, Hkv);
  if (Hq > APB_MAX_Q_HEADS)
    return fail(APB_ERR_UNSUPPORTED, "n_q_heads = %d exceeds %d", Hq, APB_MAX_Q_HEADS);
  if (pr->head_dim != 64 && pr->head_dim != 128)
    return fail(APB_ERR_UNSUPPORTED, "head_dim = %d, supported: 64, 128", pr->head_dim);
  if (pr->local_len < 1) return fail(APB_ERR_INVALID_ARGUMENT, "local_len = %d, need >= 1", pr->local_len);
  if (pr->local_len > APB_MAX_LOCAL_LEN)
    return fail(APB_ERR_UNSUPPORTED, "local_len = %d exceeds %d", pr->local_len, APB_MAX_LOCAL_LEN);
  if (pr->anchor_len < 0) return fail(APB_ERR_INVALID_ARGUMENT, "anchor_len = %d < 0", pr->anchor_len);
  if (pr->anchor_len > APB_MAX_LOCAL_LEN)
    return fail(APB_ERR_UNSUPPORTED, "anchor_len = %d exceeds %d", pr->anchor_len, APB_MAX_LOCAL_LEN);
  if (pr->n_hosts < 1) return fail(APB_ERR_INVALID_ARGUMENT, "n_hosts = %d, need >= 1", pr->n_hosts);
  if (pr->host_index < 0 || pr->host_index >= pr->n_hosts)
    return fail(APB_ERR_INVALID_ARGUMENT, "host_index = %d outside [0, %d)", pr->host_index, pr->n_hosts);
  if (pr->pass_per_host < 0 || pr->pass_per_host > pr->local_len)
    return fail(APB_ERR_INVALID_ARGUMENT, "pass_per_host = %d outside [0, local_len = %d]", pr->pass_per_host,
                pr->local_len);
  const long long P = (long long)pr->host_index * pr->pass_per_host;
  if (P > APB_MAX_LOCAL_LEN)
    return fail(APB_ERR_UNSUPPORTED, "passing length %lld exceeds %d", P, APB_MAX_LOCAL_LEN);
  if (pr->kv_head_of_q != nullptr) {
    const int g = Hq / Hkv;
    int count[APB_MAX_Q_HEADS] = {0};
    for (int i = 0; i < Hq; ++i) {
      const int h = pr->kv_head_of_q[i];
      if (h < 0 || h >= Hkv)
        return fail(APB_ERR_INVALID_ARGUMENT, "kv_head_of_q[%d] = %d outside [0, %d)", i, h, Hkv);
      ++count[h];
    }
    for (int h = 0; h < Hkv; ++h)
      if (count[h] != g)
        return fail(APB_ERR_INVALID_ARGUMENT, "kv head %d has %d q heads, need exactly %d", h, count[h], g);
  }
  return APB_OK;
}

void slot_table(const apb_problem *pr, uint8_t *out) {
  const int Hq = pr->n_q_heads, Hkv = pr->n_kv_heads, g = Hq / Hkv;
  int fill[APB_MAX_Q_HEADS] = {0};
  for (int i = 0; i < Hq; ++i) {
    const int h = pr->kv_head_of_q ? pr->kv_head_of_q[i] : i / g;
    out[h * g + fill[h]++] = (uint8_t)i;
  }
}

}  // namespace apb_host

extern "C" {

apb_status apb_validate_problem(const apb_problem *problem) {
  apb_host::clear_error();
  return apb_host::check_problem(problem);
}

const char *apb_status_string(apb_status st) {
  switch (st) {
    case APB_OK: return "APB_OK";
    case APB_ERR_INVALID_ARGUMENT: return "APB_ERR_INVALID_ARGUMENT";
    case APB_ERR_UNSUPPORTED: return "APB_ERR_UNSUPPORTED";
    case APB_ERR_WORKSPACE_TOO_SMALL: return "APB_ERR_WORKSPACE_TOO_SMALL";
    case APB_ERR_HIP: return "APB_ERR_HIP";
    case APB_ERR_INTERNAL: return "APB_ERR_INTERNAL";
  }
  return "APB_ERR_UNKNOWN";
}

const char *apb_last_error(void) { return apb_host::g_err; }

int apb_abi_version(void) { return APB_ABI_VERSION; }

}  // extern "C"
