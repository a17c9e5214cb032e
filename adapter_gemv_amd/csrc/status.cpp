// Status strings of the C ABI (host code; built into liblora_gemv.so and
// into the sanitizer build of the host-only calls).
#include "lora_gemv.h"

const char *lora_status_string(lora_status_t status) {
  switch (status) {
    case LORA_OK: return "LORA_OK";
    case LORA_ERR_NULL: return "LORA_ERR_NULL: a required pointer is NULL";
    case LORA_ERR_SHAPE: return "LORA_ERR_SHAPE: a size or leading dimension is out of range";
    case LORA_ERR_RANK: return "LORA_ERR_RANK: max_rank outside [1, LORA_MAX_RANK]";
    case LORA_ERR_ALIGN: return "LORA_ERR_ALIGN: pointer or dimension not 16-byte / 8-element aligned";
    case LORA_ERR_WORKSPACE: return "LORA_ERR_WORKSPACE: workspace too small";
    case LORA_ERR_MODULE: return "LORA_ERR_MODULE: bad module index, n_mod or module mask";
    case LORA_ERR_LAUNCH: return "LORA_ERR_LAUNCH: kernel launch failed";
    case LORA_ERR_SCRATCH:
      return "LORA_ERR_SCRATCH: the call needs more scratch than LORA_STATIC_SCRATCH_BYTES";
  }
  return "unknown lora_status_t";
}
