// pa_prefill_chunk: placeholder until the MFMA kernel lands.
#include "pa.h"
#include "pa_common.h"
#include "pa_internal.h"

extern "C" int pa_prefill_chunk(void*, float*, const void*, const int32_t*, int32_t, int32_t,
                                const void*, int32_t, const int32_t*, int32_t, const int32_t*,
                                int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, float,
                                int32_t, void*) {
  return pa::fail(PA_ENOTSUP, "pa_prefill_chunk: not built yet");
}
