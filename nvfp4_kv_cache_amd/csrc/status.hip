// status.hip -- status strings of the C ABI.
#include "msa_nvfp4.h"

extern "C" const char* msa_status_string(int32_t status) {
  switch (status) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG: null pointer, bad size or misaligned buffer";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED: shape not implemented by this library";
    case MSA_ERR_WORKSPACE: return "MSA_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case MSA_ERR_HIP: return "MSA_ERR_HIP: the HIP runtime refused a kernel launch";
  }
  return "unknown msa_status";
}
