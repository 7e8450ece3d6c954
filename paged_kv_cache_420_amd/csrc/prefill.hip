// Causal chunked prefill against the paged cache (KV-cache article,
// intelliparadigm, §4.1/§4.2: long prompts are processed in chunks).
// The matrix-core kernel is not in this build yet: the entry point exists
// so the C ABI is complete, and reports PKV_ERR_UNSUPPORTED.
#include <hip/hip_runtime.h>

#include "common.h"

using namespace pkv;

extern "C" int32_t pkv_paged_attention_prefill(
    const void*, const void*, const void*, const int32_t*, const int32_t*,
    const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t,
    int32_t, int32_t, float, float*, int32_t, void*) {
  return fail(PKV_ERR_UNSUPPORTED, "chunked prefill is not built yet");
}
