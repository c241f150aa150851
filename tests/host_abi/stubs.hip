// Host-only stand-ins for everything the C-ABI layer (abi.hip) calls below
// it: the kernel launchers and the few HIP runtime functions it uses.  Built
// with --cuda-host-only together with abi.hip and lm_codebook.hip under
// AddressSanitizer and UndefinedBehaviorSanitizer, so that every entry point's
// validation and dispatch runs on the CPU with no GPU and no HIP runtime.
// Each launcher only records that it was reached (and the output pointer it
// was handed) and returns hipSuccess, or the error the driver asked for.
#include <cstring>

#include "oq_internal.h"
#include "stubs.h"

StubState g_stub;

static hipError_t rec(const char *name, const void *out) {
  if (g_stub.launches++ == 0) g_stub.first_out = out;
  g_stub.last = name;
  g_stub.last_out = out;
  if (g_stub.fail_next) {
    g_stub.fail_next = 0;
    return hipErrorInvalidValue;
  }
  return hipSuccess;
}

namespace oq {

// the same admissible widths as the row-per-wavefront kernel's host check
bool rpbh_wave_supported(int d) { return d >= 16 && d <= 4096 && d % 16 == 0; }
int probe_blocks() { return 512; }

hipError_t launch_rpbh_quant(const uint16_t *, int64_t, int, int64_t, const RotArgs &, int, float *, int, int,
                             void *out, int64_t, float *, hipStream_t, const PctlArgs *, const LmArgs *, uint32_t *) {
  return rec("rpbh_quant", out);
}
hipError_t launch_dense32(const uint16_t *, int64_t, int, int64_t, const uint16_t *, int, void *out, int64_t,
                          uint8_t *, hipStream_t) {
  return rec("dense32", out);
}
hipError_t launch_gemm_int(const void *, int64_t, int, const float *, int64_t, int, const uint8_t *, const float *,
                           int, int, const float *, const float *, const float *, uint16_t *y, int64_t, hipStream_t,
                           void *, size_t) {
  return rec("gemm_int", y);
}
hipError_t launch_gemm_fp6(const uint8_t *, int, const float *, int64_t, int, const uint8_t *, const float *, int,
                           const float *, const float *, const float *, uint16_t *y, int64_t, hipStream_t) {
  return rec("gemm_fp6", y);
}
hipError_t launch_prepack_w4(const uint8_t *, const float *, int, int, uint8_t *out, float *, hipStream_t) {
  return rec("prepack_w4", out);
}
hipError_t launch_gemm_fp6_asym(const uint8_t *, const float *, const uint32_t *, int64_t, int, const uint8_t *,
                                const float *, const uint32_t *, int, const float *, const float *, const float *,
                                uint16_t *y, int64_t, hipStream_t) {
  return rec("gemm_fp6_asym", y);
}
hipError_t launch_prepack_w4a(const uint8_t *, const uint16_t *, const uint16_t *, int, int, uint8_t *out, float *,
                              uint32_t *, hipStream_t) {
  return rec("prepack_w4a", out);
}
hipError_t launch_gemm_mx(int, const uint8_t *, int64_t, const uint8_t *, int64_t, int, const uint8_t *,
                          const uint8_t *, int, const float *, uint16_t *y, int64_t, hipStream_t) {
  return rec("gemm_mx", y);
}
hipError_t launch_prepack_mx(const uint8_t *, const uint8_t *, int, int, uint8_t *out, uint8_t *, hipStream_t) {
  return rec("prepack_mx", out);
}
hipError_t launch_gemm_f16(const uint8_t *, const float *, int64_t, int, const uint8_t *, int, const float *,
                           const float *, const float *, uint16_t *y, int64_t, hipStream_t) {
  return rec("gemm_f16", y);
}
hipError_t launch_prepack_w16(const uint8_t *, const float *, int, int, int, uint8_t *out, hipStream_t) {
  return rec("prepack_w16", out);
}
hipError_t launch_lm_expand(const uint8_t *, int64_t, int, const uint16_t *, int, int64_t, int, uint8_t *out,
                            hipStream_t) {
  return rec("lm_expand", out);
}
hipError_t launch_weight_rpbh(const float *, int, int, int64_t, const RotArgs &, int, uint8_t *codes, float *,
                              float *, hipStream_t) {
  return rec("weight_rpbh", codes);
}
hipError_t launch_weight_rpbh_asym(const float *, int, int, int64_t, const RotArgs &, int, uint8_t *codes,
                                   uint16_t *, uint16_t *, float *, hipStream_t) {
  return rec("weight_rpbh_asym", codes);
}
hipError_t launch_weight_dense32(const float *, int, int, int64_t, const uint16_t *, uint8_t *codes, uint8_t *,
                                 float *, hipStream_t) {
  return rec("weight_dense32", codes);
}
hipError_t launch_mfma_probe(int, int, float *sink, hipStream_t, double *ops) {
  *ops = 1.0;
  return rec("mfma_probe", sink);
}

}  // namespace oq

// ----------------------------------------------------------- HIP runtime
alignas(256) static unsigned char g_fake_scratch[256];

extern "C" {

hipError_t hipGetDevice(int *dev) {
  if (g_stub.fail_get_device) return hipErrorNoDevice;
  *dev = g_stub.device;
  return hipSuccess;
}

const char *hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stub HIP error"; }

hipError_t hipGetSymbolAddress(void **p, const void *) {
  g_stub.symbol_lookups++;
  *p = g_fake_scratch;  // a 256-byte aligned stand-in address, never dereferenced
  g_stub.scratch_addr = *p;
  return hipSuccess;
}

void **__hipRegisterFatBinary(const void *) {
  static void *handle = nullptr;
  return &handle;
}
void __hipUnregisterFatBinary(void **) {}
void __hipRegisterVar(void **, void *, char *, const char *, int, size_t, int, int) {}

}  // extern "C"
