// Multi-query verify attention on MFMA (gfx950): placeholder until the MFMA
// path lands; every shape goes to the VALU kernel.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

bool verify_mfma_supported(const DecodeArgs&) { return false; }

hipError_t launch_verify_mfma(const DecodeArgs&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace pkv
