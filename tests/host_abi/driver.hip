// Validation driver for the C ABI on the CPU: every entry point of oq.h is
// called with well-formed arguments (expect OQ_OK and the launchers it
// dispatches to) and with each kind of malformed argument its header names
// (expect the documented OQ_ERR_* code and no launch at all).  Pointers are
// host addresses that the stand-in launchers never dereference; host-side
// outputs (Lloyd-Max tables, the Kronecker plan) are real and checked.
// Prints "<n> cases passed" and exits 0, or lists each failure and exits 1.
#include <cmath>
#include <cstdio>
#include <cstring>

#include "oq.h"
#include "stubs.h"

namespace {

int g_cases = 0, g_fail = 0;

alignas(256) unsigned char g_buf[1 << 16];
unsigned char *P = g_buf;        // 256-byte aligned
unsigned char *Q = g_buf + 1;    // misaligned by one byte
unsigned char *Q4 = g_buf + 4;   // 4-byte but not 16-byte aligned
int32_t g_perm[8];
int8_t g_signs[8];

void reset() {
  g_stub.launches = 0;
  g_stub.first_out = nullptr;
  g_stub.last = "";
  g_stub.last_out = nullptr;
  g_stub.fail_next = 0;
  g_stub.fail_get_device = 0;
}

void expect(int line, const char *what, int rc, int code, int launches) {
  ++g_cases;
  if (rc != code || g_stub.launches != launches) {
    ++g_fail;
    std::printf("line %d: %s -> rc %d (want %d), launches %d (want %d), last error '%s'\n", line, what, rc, code,
                g_stub.launches, launches, oq_last_error());
  } else if (rc != OQ_OK && oq_last_error()[0] == 0) {
    ++g_fail;
    std::printf("line %d: %s -> rc %d with an empty error message\n", line, what, rc);
  }
  reset();
}

void truth(int line, const char *what, bool ok) {
  ++g_cases;
  if (!ok) {
    ++g_fail;
    std::printf("line %d: %s is false\n", line, what);
  }
}

#define EXPECT(call, code, launches) expect(__LINE__, #call, (call), (code), (launches))
#define TRUE(cond) truth(__LINE__, #cond, (cond))

const uint16_t *X = reinterpret_cast<const uint16_t *>(g_buf);
float *F = reinterpret_cast<float *>(g_buf);
uint16_t *Y = reinterpret_cast<uint16_t *>(g_buf);

oq_rot rpbh(int d, int block, int rounds) { return oq_rot{OQ_ROT_RPBH, d, block, rounds, g_perm, g_signs, nullptr}; }
oq_rot dense(int d) { return oq_rot{OQ_ROT_DENSE32, d, 32, 1, nullptr, nullptr, reinterpret_cast<const uint16_t *>(P)}; }
oq_rot kron(int d, int m, int block) { return oq_rot{OQ_ROT_KRON, d, block, m, nullptr, nullptr, nullptr}; }

void center_rotate() {
  EXPECT(oq_center(X, 4, 64, 64, F, 64, F, nullptr), OQ_OK, 1);
  EXPECT(oq_center(X, 4, 64, 64, nullptr, 0, F, nullptr), OQ_OK, 1);
  EXPECT(oq_center(X, -1, 64, 64, F, 64, F, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_center(nullptr, 4, 64, 64, F, 64, F, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_center(X, 4, 8, 64, F, 64, F, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_center(X, 4, 20000, 20000, F, 20000, F, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_center(X, 4, 72, 72, F, 72, F, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_center(X, 4, 64, 32, F, 64, F, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_center(reinterpret_cast<const uint16_t *>(Q), 4, 64, 64, F, 64, F, nullptr), OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_center(X, 4, 64, 68, F, 64, F, nullptr), OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_center(X, 4, 64, 64, F, 64, nullptr, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_center(X, 4, 64, 64, reinterpret_cast<float *>(Q4), 64, F, nullptr), OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_center(X, 4, 64, 64, F, 63, F, nullptr), OQ_ERR_ALIGNMENT, 0);

  oq_rot r = rpbh(256, 128, 1);
  EXPECT(oq_rotate(&r, X, 4, 256, 0, nullptr, F, 256, nullptr), OQ_OK, 1);
  EXPECT(oq_rotate(nullptr, X, 4, 256, 0, nullptr, F, 256, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_rotate(&r, X, 4, 256, 1, nullptr, F, 256, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_rotate(&r, X, 4, 256, 0, nullptr, nullptr, 256, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_rotate(&r, X, 4, 256, 0, nullptr, F, 128, nullptr), OQ_ERR_ALIGNMENT, 0);
  r = rpbh(256, 48, 1);
  EXPECT(oq_rotate(&r, X, 4, 256, 0, nullptr, F, 256, nullptr), OQ_ERR_UNSUPPORTED, 0);
  r = rpbh(4096, 2048, 1);
  EXPECT(oq_rotate(&r, X, 4, 4096, 0, nullptr, F, 4096, nullptr), OQ_ERR_UNSUPPORTED, 0);
  r = rpbh(256, 16, 1);
  EXPECT(oq_rotate(&r, X, 4, 256, 0, nullptr, F, 256, nullptr), OQ_ERR_UNSUPPORTED, 0);
  r = rpbh(256, 128, 3);
  EXPECT(oq_rotate(&r, X, 4, 256, 0, nullptr, F, 256, nullptr), OQ_ERR_UNSUPPORTED, 0);
  r = rpbh(256, 128, 0);
  EXPECT(oq_rotate(&r, X, 4, 256, 0, nullptr, F, 256, nullptr), OQ_ERR_UNSUPPORTED, 0);
  r = rpbh(192, 128, 1);
  EXPECT(oq_rotate(&r, X, 4, 192, 0, nullptr, F, 192, nullptr), OQ_ERR_INVALID_ARG, 0);
  r = rpbh(256, 128, 1);
  r.perm = nullptr;
  EXPECT(oq_rotate(&r, X, 4, 256, 0, nullptr, F, 256, nullptr), OQ_ERR_INVALID_ARG, 0);
  r = rpbh(256, 128, 1);
  r.kind = 9;
  EXPECT(oq_rotate(&r, X, 4, 256, 0, nullptr, F, 256, nullptr), OQ_ERR_INVALID_ARG, 0);

  oq_rot dr = dense(256);
  EXPECT(oq_rotate(&dr, X, 4, 256, 0, nullptr, F, 256, nullptr), OQ_OK, 1);
  EXPECT(oq_rotate(&dr, X, 4, 256, 1, F, F, 256, nullptr), OQ_ERR_UNSUPPORTED, 0);
  dr.mats = nullptr;
  EXPECT(oq_rotate(&dr, X, 4, 256, 0, nullptr, F, 256, nullptr), OQ_ERR_INVALID_ARG, 0);
  dr.mats = reinterpret_cast<const uint16_t *>(Q4);
  EXPECT(oq_rotate(&dr, X, 4, 256, 0, nullptr, F, 256, nullptr), OQ_ERR_ALIGNMENT, 0);
  dr = dense(48);
  EXPECT(oq_rotate(&dr, X, 4, 48, 0, nullptr, F, 48, nullptr), OQ_ERR_INVALID_ARG, 0);

  oq_rot kr = kron(368, 12, 32);  // padded width 384
  EXPECT(oq_rotate(&kr, X, 4, 368, 0, nullptr, F, 384, nullptr), OQ_OK, 1);
  EXPECT(oq_rotate(&kr, X, 4, 368, 0, nullptr, F, 368, nullptr), OQ_ERR_ALIGNMENT, 0);
  kr = kron(368, 5, 128);
  EXPECT(oq_rotate(&kr, X, 4, 368, 0, nullptr, F, 640, nullptr), OQ_ERR_UNSUPPORTED, 0);
  kr = kron(400, 12, 32);
  EXPECT(oq_rotate(&kr, X, 4, 400, 0, nullptr, F, 400, nullptr), OQ_ERR_UNSUPPORTED, 0);
  kr = kron(368, 12, 24);
  EXPECT(oq_rotate(&kr, X, 4, 368, 0, nullptr, F, 384, nullptr), OQ_ERR_UNSUPPORTED, 0);
}

void quant_act() {
  oq_rot r = rpbh(256, 128, 1);
  EXPECT(oq_quant_act(X, 4, 256, 256, &r, 0, OQ_A8, P, 256, F, nullptr, nullptr, nullptr), OQ_OK, 1);
  EXPECT(oq_quant_act(X, 4, 256, 256, nullptr, 0, OQ_A8, P, 256, F, nullptr, nullptr, nullptr), OQ_OK, 1);
  EXPECT(oq_quant_act(X, 4, 256, 256, &r, 1, OQ_A4, P, 128, F, nullptr, F, nullptr), OQ_OK, 1);
  EXPECT(oq_quant_act(X, 4, 256, 256, &r, 0, OQ_A4, P, 112, F, nullptr, nullptr, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_quant_act(X, 4, 256, 256, &r, 0, OQ_A8, P, 264, F, nullptr, nullptr, nullptr), OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_quant_act(X, 4, 256, 256, &r, 0, OQ_A8, Q, 256, F, nullptr, nullptr, nullptr), OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_quant_act(X, 4, 256, 256, &r, 0, OQ_A8, nullptr, 256, F, nullptr, nullptr, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_quant_act(X, 4, 256, 256, &r, 0, OQ_A8, P, 256, nullptr, nullptr, nullptr, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_quant_act(X, 4, 256, 256, &r, 1, OQ_A8, P, 256, F, nullptr, nullptr, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_quant_act(X, 4, 256, 256, &r, 0, OQ_A8, P, 256, F, P, nullptr, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_quant_act(X, 4, 256, 256, &r, 0, 77, P, 256, F, nullptr, nullptr, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_quant_act(X, 4, 256, 256, &r, 0, OQ_A4 | OQ_TILED, P, 0, F, nullptr, nullptr, nullptr), OQ_OK, 1);
  EXPECT(oq_quant_act(X, 4, 256, 256, &r, 0, OQ_A6 | OQ_TILED, P, 0, F, nullptr, nullptr, nullptr), OQ_OK, 1);
  EXPECT(oq_quant_act(X, 4, 256, 256, &r, 0, OQ_A8 | OQ_TILED, P, 0, F, nullptr, nullptr, nullptr), OQ_ERR_UNSUPPORTED, 0);
  oq_rot r96 = rpbh(96, 32, 1);
  EXPECT(oq_quant_act(X, 4, 96, 96, &r96, 0, OQ_A4 | OQ_TILED, P, 0, F, nullptr, nullptr, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_quant_act(X, 4, 256, 256, &r, 0, OQ_A4 | OQ_TILED | OQ_SCALE_PCTL, P, 0, F, nullptr, nullptr, nullptr), OQ_OK, 1);
  EXPECT(oq_quant_act(X, 4, 8192, 8192, nullptr, 0, OQ_A4 | OQ_SCALE_PCTL, P, 4096, F, nullptr, nullptr, nullptr),
         OQ_ERR_UNSUPPORTED, 0);
  oq_rot kr = kron(368, 12, 32);
  EXPECT(oq_quant_act(X, 4, 368, 368, &kr, 0, OQ_A8, P, 384, F, nullptr, nullptr, nullptr), OQ_OK, 1);
  EXPECT(oq_quant_act(X, 4, 368, 368, &kr, 0, OQ_A8, P, 368, F, nullptr, nullptr, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_quant_act(X, 4, 368, 368, &kr, 0, OQ_A8 | OQ_SCALE_PCTL, P, 384, F, nullptr, nullptr, nullptr),
         OQ_ERR_UNSUPPORTED, 0);

  oq_rot dr = dense(256);
  uint8_t *E = P + 4096;
  EXPECT(oq_quant_act(X, 4, 256, 256, &dr, 0, OQ_MXFP4 | OQ_TILED, P, 0, nullptr, E, nullptr, nullptr), OQ_OK, 1);
  EXPECT(oq_quant_act(X, 4, 256, 256, &dr, 0, OQ_MXFP4, P, 128, nullptr, E, nullptr, nullptr), OQ_OK, 1);
  EXPECT(oq_quant_act(X, 4, 256, 256, &dr, 0, OQ_MXFP4, P, 112, nullptr, E, nullptr, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_quant_act(X, 4, 256, 256, &dr, 0, OQ_MXFP4 | OQ_TILED, P, 0, F, E, nullptr, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_quant_act(X, 4, 256, 256, &dr, 0, OQ_MXFP4 | OQ_TILED, P, 0, nullptr, nullptr, nullptr, nullptr),
         OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_quant_act(X, 4, 256, 256, &dr, 0, OQ_MXFP4 | OQ_TILED, P, 0, nullptr, Q, nullptr, nullptr), OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_quant_act(X, 4, 256, 256, &dr, 1, OQ_MXFP4 | OQ_TILED, P, 0, nullptr, E, F, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_quant_act(X, 4, 256, 256, &r, 0, OQ_MXFP4 | OQ_TILED, P, 0, nullptr, E, nullptr, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_quant_act(X, 4, 256, 256, &r, 0, OQ_MXFP4, P, 128, nullptr, E, nullptr, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_quant_act(X, 4, 256, 256, &dr, 0, OQ_A8, P, 256, F, nullptr, nullptr, nullptr), OQ_ERR_INVALID_ARG, 0);
  oq_rot d160 = dense(160);
  EXPECT(oq_quant_act(X, 4, 160, 160, &d160, 0, OQ_MXFP4 | OQ_TILED, P, 0, nullptr, E, nullptr, nullptr),
         OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_quant_act(X, 4, 256, 256, &dr, 0, OQ_MXFP4 | OQ_SCALE_PCTL, P, 128, nullptr, E, nullptr, nullptr),
         OQ_ERR_UNSUPPORTED, 0);
  // empty batch: validated, dispatched with M = 0 (the launchers return at once)
  EXPECT(oq_quant_act(nullptr, 0, 256, 256, &r, 0, OQ_A8, nullptr, 256, nullptr, nullptr, nullptr, nullptr), OQ_OK, 1);
}

void quant_weight_prepack() {
  oq_rot r = rpbh(256, 128, 1);
  EXPECT(oq_quant_weight(F, 64, 256, 256, &r, OQ_W4, 64, P, F, F, nullptr), OQ_OK, 1);
  EXPECT(oq_quant_weight(F, 64, 256, 256, nullptr, OQ_W4, 128, P, F, nullptr, nullptr), OQ_OK, 1);
  EXPECT(oq_quant_weight(F, -1, 256, 256, &r, OQ_W4, 64, P, F, F, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_quant_weight(F, 64, 40, 40, nullptr, OQ_W4, 32, P, F, F, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_quant_weight(F, 64, 32768, 32768, nullptr, OQ_W4, 64, P, F, F, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_quant_weight(F, 64, 256, 128, &r, OQ_W4, 64, P, F, F, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_quant_weight(F, 64, 256, 258, &r, OQ_W4, 64, P, F, F, nullptr), OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_quant_weight(F, 64, 256, 256, &r, OQ_W4, 48, P, F, F, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_quant_weight(F, 64, 256, 256, &r, OQ_W4, 512, P, F, F, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_quant_weight(F, 64, 256, 256, &r, 5, 64, P, F, F, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_quant_weight(F, 64, 256, 256, &r, OQ_W4, 64, nullptr, F, F, nullptr), OQ_ERR_INVALID_ARG, 0);
  oq_rot dr = dense(256);
  EXPECT(oq_quant_weight(F, 64, 256, 256, &dr, OQ_W_MXFP4, 32, P, P, nullptr, nullptr), OQ_OK, 1);
  EXPECT(oq_quant_weight(F, 64, 256, 256, &dr, OQ_W_MXFP4, 32, P, P, F, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_quant_weight(F, 64, 256, 256, &r, OQ_W_MXFP4, 32, P, P, nullptr, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_quant_weight(F, 64, 256, 256, &dr, OQ_W4, 64, P, F, nullptr, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_quant_weight(nullptr, 0, 256, 256, &r, OQ_W4, 64, nullptr, nullptr, nullptr, nullptr), OQ_OK, 1);

  EXPECT(oq_prepack_w4(P, F, 64, 256, 64, P, F, nullptr), OQ_OK, 1);
  EXPECT(oq_prepack_w4(P, F, 64, 256, 32, P, F, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_prepack_w4(P, F, 64, 96, 64, P, F, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_prepack_w4(P, F, -2, 256, 64, P, F, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_prepack_w4(P, F, 64, 256, 64, nullptr, F, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_prepack_w4(Q, F, 64, 256, 64, P, F, nullptr), OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_prepack_mx(P, P, 64, 256, P, P, nullptr), OQ_OK, 1);
  EXPECT(oq_prepack_mx(P, P, 64, 192, P, P, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_prepack_mx(P, P, 64, 256, P, Q, nullptr), OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_prepack_mx(P, nullptr, 64, 256, P, P, nullptr), OQ_ERR_INVALID_ARG, 0);

  // sizes of the tiled layouts: rows padded to 32; 48 bytes per row and 64
  // codes (FP6), 32 bytes per row and 64 codes (E2M1)
  TRUE(oq_tiled_bytes(33, 128) == 64 * 96);
  TRUE(oq_tiled_bytes(-1, 128) == 0);
  TRUE(oq_tiled_mx_bytes(33, 128) == 64 * 64);
  TRUE(oq_tiled_f16_bytes(33, 128) == 64 * 256);
  TRUE(oq_tiled_f16_bytes(33, 120) == 0);
}

void gemms() {
  const float *S = F;
  EXPECT(oq_gemm_w4a8(reinterpret_cast<const int8_t *>(P), 256, S, 5, 256, P, S, 64, 128, nullptr, nullptr, nullptr, Y,
                      64, nullptr, 0, nullptr), OQ_OK, 1);
  EXPECT(oq_gemm_w4a8(reinterpret_cast<const int8_t *>(P), 256, S, 5, 256, P, S, 64, 128, S, S, S, Y, 64, nullptr, 0,
                      nullptr), OQ_OK, 1);
  EXPECT(oq_gemm_w4a8(reinterpret_cast<const int8_t *>(P), 256, S, 5, 100, P, S, 64, 128, nullptr, nullptr, nullptr, Y,
                      64, nullptr, 0, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_gemm_w4a8(reinterpret_cast<const int8_t *>(P), 128, S, 5, 256, P, S, 64, 128, nullptr, nullptr, nullptr, Y,
                      64, nullptr, 0, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_gemm_w4a8(reinterpret_cast<const int8_t *>(P), 264, S, 5, 256, P, S, 64, 128, nullptr, nullptr, nullptr, Y,
                      64, nullptr, 0, nullptr), OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_gemm_w4a8(reinterpret_cast<const int8_t *>(P), 256, S, 5, 256, P, S, 64, 128, nullptr, nullptr, nullptr, Y,
                      32, nullptr, 0, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_gemm_w4a8(reinterpret_cast<const int8_t *>(P), 256, S, 5, 256, P, S, 64, 128, nullptr, nullptr, nullptr,
                      reinterpret_cast<uint16_t *>(Q), 64, nullptr, 0, nullptr), OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_gemm_w4a8(reinterpret_cast<const int8_t *>(P), 256, S, 5, 256, P, S, 64, 128, S, nullptr, nullptr, Y, 64,
                      nullptr, 0, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_gemm_w4a8(reinterpret_cast<const int8_t *>(P), 256, S, 5, 256, P, S, 64, 48, nullptr, nullptr, nullptr, Y,
                      64, nullptr, 0, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_gemm_w4a8(reinterpret_cast<const int8_t *>(P), 256, nullptr, 5, 256, P, S, 64, 128, nullptr, nullptr,
                      nullptr, Y, 64, nullptr, 0, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_gemm_w4a8(reinterpret_cast<const int8_t *>(P), 256, S, -5, 256, P, S, 64, 128, nullptr, nullptr, nullptr, Y,
                      64, nullptr, 0, nullptr), OQ_ERR_INVALID_ARG, 0);
  // optional split scratch: none for a small product with K <= 4096 (the 32
  // x 32 tile kernel); beyond, one 128 x 128 tile splits into min(256, K /
  // 32) = 256 parts
  TRUE(oq_workspace_bytes(OQ_OP_GEMM_W4A8, 5, 256, 64, 0) == 0);
  TRUE(oq_workspace_bytes(OQ_OP_GEMM_W4A8, 5, 8192, 64, 0) == 256u * 5 * 64 * 4);
  TRUE(oq_workspace_bytes(OQ_OP_GEMM_W4A8, 2048, 256, 2048, 0) == 0);  // 256 tiles: one pass
  TRUE(oq_workspace_bytes(OQ_OP_GEMM_W4A8, 5, 256, 0, 0) == 0);
  EXPECT(oq_gemm_w4a8(reinterpret_cast<const int8_t *>(P), 256, S, 5, 256, P, S, 64, 128, nullptr, nullptr, nullptr, Y,
                      64, P, 10240, nullptr), OQ_OK, 1);
  EXPECT(oq_gemm_w4a8(reinterpret_cast<const int8_t *>(P), 256, S, 5, 256, P, S, 64, 128, nullptr, nullptr, nullptr, Y,
                      64, Q4, 10240, nullptr), OQ_ERR_ALIGNMENT, 0);

  EXPECT(oq_gemm_w4a4(OQ_A4 | OQ_TILED, P, 0, S, 5, 256, P, S, 64, 64, nullptr, nullptr, nullptr, Y, 64, nullptr, 0,
                      nullptr), OQ_OK, 1);
  EXPECT(oq_gemm_w4a4(OQ_A6 | OQ_TILED, P, 0, S, 5, 256, P, S, 64, 64, S, S, nullptr, Y, 64, nullptr, 0, nullptr),
         OQ_OK, 1);
  EXPECT(oq_gemm_w4a4(OQ_A8 | OQ_TILED, P, 0, S, 5, 256, P, S, 64, 64, nullptr, nullptr, nullptr, Y, 64, nullptr, 0,
                      nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_gemm_w4a4(OQ_A4 | OQ_TILED, P, 0, S, 5, 256, P, S, 64, 32, nullptr, nullptr, nullptr, Y, 64, nullptr, 0,
                      nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_gemm_w4a4(OQ_A4 | OQ_TILED, P, 0, nullptr, 5, 256, P, S, 64, 64, nullptr, nullptr, nullptr, Y, 64, nullptr,
                      0, nullptr), OQ_ERR_INVALID_ARG, 0);
  // 400000 rows of K = 16384 make an operand plane beyond 4 GiB
  EXPECT(oq_gemm_w4a4(OQ_A4 | OQ_TILED, P, 0, S, 400000, 16384, P, S, 64, 64, nullptr, nullptr, nullptr, Y, 64, nullptr,
                      0, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_gemm_w4a4(OQ_A4 | OQ_TILED, P, 0, S, 64, 16384, P, S, 400000, 64, nullptr, nullptr, nullptr, Y, 400000,
                      nullptr, 0, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_gemm_w4a4(OQ_MXFP4 | OQ_TILED, P, 0, P, 5, 256, P, P, 64, 32, nullptr, nullptr, nullptr, Y, 64, nullptr, 0,
                      nullptr), OQ_OK, 1);
  EXPECT(oq_gemm_w4a4(OQ_MXFP4 | OQ_TILED, P, 0, P, 5, 256, P, P, 64, 64, nullptr, nullptr, nullptr, Y, 64, nullptr, 0,
                      nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_gemm_w4a4(OQ_MXFP4 | OQ_TILED, P, 0, P, 5, 192, P, P, 64, 32, nullptr, nullptr, nullptr, Y, 64, nullptr, 0,
                      nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_gemm_w4a4(OQ_MXFP4 | OQ_TILED, P, 0, P, 5, 256, P, P, 64, 32, S, S, nullptr, Y, 64, nullptr, 0, nullptr),
         OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_gemm_w4a4(OQ_MXFP4 | OQ_TILED, P, 0, Q, 5, 256, P, P, 64, 32, nullptr, nullptr, nullptr, Y, 64, nullptr, 0,
                      nullptr), OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_gemm_w4a4(OQ_MXFP4, P, 128, P, 5, 256, P, P, 64, 32, nullptr, nullptr, nullptr, Y, 64, nullptr, 0, nullptr),
         OQ_OK, 1);
  EXPECT(oq_gemm_w4a4(OQ_A4, P, 128, S, 5, 256, P, S, 64, 64, nullptr, nullptr, nullptr, Y, 64, nullptr, 0, nullptr),
         OQ_OK, 1);
  EXPECT(oq_gemm_w4a4(OQ_A4, P, 112, S, 5, 256, P, S, 64, 64, nullptr, nullptr, nullptr, Y, 64, nullptr, 0, nullptr),
         OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_gemm_w4a4(OQ_A6, P, 256, S, 5, 256, P, S, 64, 64, nullptr, nullptr, nullptr, Y, 64, nullptr, 0, nullptr),
         OQ_ERR_INVALID_ARG, 0);
  // an empty product passes validation with NULL operands (the launcher returns at once)
  EXPECT(oq_gemm_w4a4(OQ_A4 | OQ_TILED, nullptr, 0, nullptr, 0, 256, nullptr, nullptr, 64, 64, nullptr, nullptr, nullptr,
                      nullptr, 64, nullptr, 0, nullptr), OQ_OK, 1);
}

void fused() {
  oq_rot r = rpbh(256, 128, 1);
  const size_t ws_t = oq_workspace_bytes(OQ_OP_LINEAR, 5, 256, 64, OQ_A4 | OQ_TILED);
  const size_t ws_8 = oq_workspace_bytes(OQ_OP_LINEAR, 5, 256, 64, OQ_A8);
  // row-major 8-bit codes: 5 rows of 256 bytes, then 5 scales and 5 means, each piece 256-aligned
  TRUE(ws_8 == 1792);
  // tiled 4-bit codes: 32 padded rows of 192 bytes, then the scales and the means
  TRUE(ws_t == 6144 + 256 + 256);
  TRUE(oq_workspace_bytes(OQ_OP_LINEAR, -1, 256, 64, OQ_A8) == 0);
  TRUE(oq_workspace_bytes(OQ_OP_GEMM_LM, 5, 256, 64, OQ_TILED) == 0);
  TRUE(oq_workspace_bytes(OQ_OP_GEMM_LM, 5, 256, 64, 0) == oq_tiled_f16_bytes(5, 256));
  TRUE(oq_workspace_bytes(OQ_OP_LINEAR, 5, 256, 64, OQ_A4 | OQ_TILED | OQ_SCALE_PCTL) == ws_t);
  const float *S = F;
  EXPECT(oq_linear_fused(X, 5, 256, 256, &r, 0, OQ_A4 | OQ_TILED, P, S, 64, 64, nullptr, nullptr, Y, 64, P, ws_t,
                         nullptr), OQ_OK, 2);
  const size_t ws_6 = oq_workspace_bytes(OQ_OP_LINEAR, 5, 256, 64, OQ_A6 | OQ_TILED);
  TRUE(ws_6 == 2 * 6144 + 256 + 256);
  EXPECT(oq_linear_fused(X, 5, 256, 256, &r, 1, OQ_A6 | OQ_TILED, P, S, 64, 64, S, S, Y, 64, P, ws_6, nullptr), OQ_OK, 2);
  EXPECT(oq_linear_fused(X, 5, 256, 256, &r, 1, OQ_A6 | OQ_TILED, P, S, 64, 64, S, S, Y, 64, P, ws_t, nullptr),
         OQ_ERR_WORKSPACE, 0);
  EXPECT(oq_linear_fused(X, 5, 256, 256, &r, 0, OQ_A4 | OQ_TILED, P, S, 64, 64, nullptr, nullptr, Y, 64, P, ws_t - 1,
                         nullptr), OQ_ERR_WORKSPACE, 0);
  EXPECT(oq_linear_fused(X, 5, 256, 256, &r, 0, OQ_A4 | OQ_TILED, P, S, 64, 64, nullptr, nullptr, Y, 64, nullptr, 0,
                         nullptr), OQ_ERR_WORKSPACE, 0);
  EXPECT(oq_linear_fused(X, 5, 256, 256, &r, 0, OQ_A4 | OQ_TILED, P, S, 64, 64, nullptr, nullptr, Y, 64, Q4, ws_t,
                         nullptr), OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_linear_fused(X, 5, 256, 256, &r, 1, OQ_A4 | OQ_TILED, P, S, 64, 64, nullptr, nullptr, Y, 64, P, ws_t,
                         nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_linear_fused(X, 5, 256, 256, &r, 0, OQ_A4 | OQ_TILED, P, S, 64, 128, nullptr, nullptr, Y, 64, P, ws_t,
                         nullptr), OQ_ERR_UNSUPPORTED, 0);
  oq_rot kr = kron(368, 12, 32);
  EXPECT(oq_linear_fused(X, 5, 368, 368, &kr, 0, OQ_A8, P, S, 64, 16, nullptr, nullptr, Y, 64, P, 1 << 14, nullptr),
         OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_linear_fused(X, 5, 256, 256, &r, 0, OQ_A8, P, S, 64, 128, nullptr, nullptr, Y, 64, P, ws_8, nullptr), OQ_OK,
         2);
  EXPECT(oq_linear_fused(X, 5, 256, 256, &r, 0, 77, P, S, 64, 128, nullptr, nullptr, Y, 64, P, ws_8, nullptr),
         OQ_ERR_INVALID_ARG, 0);
  oq_rot dr = dense(256);
  const size_t ws_m = oq_workspace_bytes(OQ_OP_LINEAR, 5, 256, 64, OQ_MXFP4 | OQ_TILED);
  EXPECT(oq_linear_fused(X, 5, 256, 256, &dr, 0, OQ_MXFP4 | OQ_TILED, P, P, 64, 32, nullptr, nullptr, Y, 64, P, ws_m,
                         nullptr), OQ_OK, 2);
  EXPECT(oq_linear_fused(X, 5, 256, 256, &dr, 1, OQ_MXFP4 | OQ_TILED, P, P, 64, 32, nullptr, nullptr, Y, 64, P, ws_m,
                         nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_linear_fused(X, 5, 256, 256, &r, 0, OQ_MXFP4 | OQ_TILED, P, P, 64, 32, nullptr, nullptr, Y, 64, P, ws_m,
                         nullptr), OQ_ERR_UNSUPPORTED, 0);
  const size_t ws_r = oq_workspace_bytes(OQ_OP_LINEAR, 5, 256, 64, OQ_MXFP4);
  EXPECT(oq_linear_fused(X, 5, 256, 256, &dr, 0, OQ_MXFP4, P, P, 64, 32, nullptr, nullptr, Y, 64, P, ws_r, nullptr),
         OQ_OK, 2);
  // a launch error becomes OQ_ERR_HIP and stops the call
  g_stub.fail_next = 1;
  EXPECT(oq_linear_fused(X, 5, 256, 256, &r, 0, OQ_A4 | OQ_TILED, P, S, 64, 64, nullptr, nullptr, Y, 64, P, ws_t,
                         nullptr), OQ_ERR_HIP, 1);

  // the entry point without a workspace: codes go to the static scratch's
  // device address, looked up once per device
  const int before = g_stub.symbol_lookups;
  EXPECT(oq_linear_fused_noalloc(X, 5, 256, 256, &r, 0, OQ_A4 | OQ_TILED, P, S, 64, 64, nullptr, nullptr, Y, 64,
                                 nullptr), OQ_OK, 2);
  g_stub.launches = 0;
  oq_linear_fused_noalloc(X, 5, 256, 256, &r, 0, OQ_A8, P, S, 64, 128, nullptr, nullptr, Y, 64, nullptr);
  TRUE(g_stub.symbol_lookups == before + 1);
  reset();
  (void)oq_linear_fused_noalloc(X, 5, 256, 256, &r, 0, OQ_A8, P, S, 64, 128, nullptr, nullptr, Y, 64, nullptr);
  TRUE(g_stub.first_out == g_stub.scratch_addr && g_stub.last_out == Y);
  reset();
  g_stub.device = 3;
  EXPECT(oq_linear_fused_noalloc(X, 5, 256, 256, &r, 0, OQ_A8, P, S, 64, 128, nullptr, nullptr, Y, 64, nullptr), OQ_OK, 2);
  TRUE(g_stub.symbol_lookups == before + 2);
  g_stub.device = 0;
  g_stub.fail_get_device = 1;
  EXPECT(oq_linear_fused_noalloc(X, 5, 256, 256, &r, 0, OQ_A8, P, S, 64, 128, nullptr, nullptr, Y, 64, nullptr),
         OQ_ERR_HIP, 0);
  g_stub.device = 64;
  EXPECT(oq_linear_fused_noalloc(X, 5, 256, 256, &r, 0, OQ_A8, P, S, 64, 128, nullptr, nullptr, Y, 64, nullptr),
         OQ_ERR_UNSUPPORTED, 0);
  g_stub.device = 0;
  EXPECT(oq_linear_fused_noalloc(X, 100000, 4096, 4096, &r, 0, OQ_A4 | OQ_TILED, P, S, 64, 64, nullptr, nullptr, Y, 64,
                                 nullptr), OQ_ERR_WORKSPACE, 0);
  EXPECT(oq_linear_fused_noalloc(X, -1, 256, 256, &r, 0, OQ_A8, P, S, 64, 128, nullptr, nullptr, Y, 64, nullptr),
         OQ_ERR_INVALID_ARG, 0);
}

void lloyd_max() {
  double lv[256];
  EXPECT(oq_lloyd_max_levels(2, 4, lv), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_lloyd_max_levels(128, 9, lv), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_lloyd_max_levels(128, 0, lv), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_lloyd_max_levels(128, 4, nullptr), OQ_ERR_INVALID_ARG, 0);
  for (int bits = 1; bits <= 8; bits += 7) {
    EXPECT(oq_lloyd_max_levels(3072, bits, lv), OQ_OK, 0);
    const int L = 1 << bits;
    bool sym = true, inc = true;
    for (int i = 0; i < L; ++i) sym = sym && lv[i] == -lv[L - 1 - i];
    for (int i = 0; i + 1 < L; ++i) inc = inc && lv[i] < lv[i + 1];
    TRUE(sym && inc);
  }
  uint16_t l16[256];
  float th[255];
  EXPECT(oq_lloyd_max_tables(4096, 8, l16, th), OQ_OK, 0);
  EXPECT(oq_lloyd_max_tables(4096, 8, nullptr, th), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_lloyd_max_tables(4096, 12, l16, th), OQ_ERR_UNSUPPORTED, 0);

  oq_rot r = rpbh(256, 128, 1);
  const float *S = F;
  const uint16_t *LV = reinterpret_cast<const uint16_t *>(P);
  EXPECT(oq_quant_act_lm(X, 4, 256, 256, &r, 0, 4, 0, LV, S, P, 128, F, nullptr, nullptr), OQ_OK, 1);
  EXPECT(oq_quant_act_lm(X, 4, 256, 256, &r, 1, 8, 1, LV, S, P, 0, F, F, nullptr), OQ_OK, 1);
  EXPECT(oq_quant_act_lm(X, 4, 8192, 8192, nullptr, 0, 4, 0, LV, S, P, 4096, F, nullptr, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_quant_act_lm(X, 4, 256, 256, &r, 0, 4, 0, nullptr, S, P, 128, F, nullptr, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_quant_act_lm(X, 4, 256, 256, &r, 0, 4, 0, reinterpret_cast<const uint16_t *>(Q), S, P, 128, F, nullptr,
                         nullptr), OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_quant_act_lm(X, 4, 256, 256, &r, 0, 8, 0, LV, S, P, 128, F, nullptr, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_quant_act_lm(X, 4, 256, 256, &r, 0, 4, 0, LV, S, P, 136, F, nullptr, nullptr), OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_quant_act_lm(X, 4, 256, 256, &r, 1, 4, 0, LV, S, P, 128, F, nullptr, nullptr), OQ_ERR_INVALID_ARG, 0);
  oq_rot kr = kron(368, 12, 32);
  EXPECT(oq_quant_act_lm(X, 4, 368, 368, &kr, 0, 4, 0, LV, S, P, 192, F, nullptr, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_quant_act_lm(nullptr, 0, 256, 256, &r, 0, 4, 0, nullptr, nullptr, nullptr, 0, nullptr, nullptr, nullptr),
         OQ_OK, 0);

  EXPECT(oq_prepack_w16(P, S, 64, 256, 64, reinterpret_cast<uint16_t *>(P), nullptr), OQ_OK, 1);
  EXPECT(oq_prepack_w16(P, S, 64, 256, 48, reinterpret_cast<uint16_t *>(P), nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_prepack_w16(P, S, 64, 240, 48, reinterpret_cast<uint16_t *>(P), nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_prepack_w16(P, S, 64, 256, 64, reinterpret_cast<uint16_t *>(Q), nullptr), OQ_ERR_ALIGNMENT, 0);

  const uint16_t *W16 = reinterpret_cast<const uint16_t *>(P);
  const size_t need = oq_workspace_bytes(OQ_OP_GEMM_LM, 5, 256, 64, 0);
  EXPECT(oq_gemm_lm(4, 0, P, 128, S, 5, 256, LV, W16, 64, nullptr, nullptr, nullptr, Y, 64, P, need, nullptr), OQ_OK, 2);
  EXPECT(oq_gemm_lm(4, 0, P, 128, S, 5, 256, LV, W16, 64, nullptr, nullptr, nullptr, Y, 64, P, need - 16, nullptr),
         OQ_ERR_WORKSPACE, 0);
  EXPECT(oq_gemm_lm(4, 0, P, 120, S, 5, 256, LV, W16, 64, nullptr, nullptr, nullptr, Y, 64, P, need, nullptr),
         OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_gemm_lm(4, 0, P, 128, S, 5, 256, nullptr, W16, 64, nullptr, nullptr, nullptr, Y, 64, P, need, nullptr),
         OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_gemm_lm(8, 1, P, 0, S, 5, 256, nullptr, W16, 64, S, S, S, Y, 64, nullptr, 0, nullptr), OQ_OK, 1);
  EXPECT(oq_gemm_lm(0, 1, P, 0, S, 5, 256, nullptr, W16, 64, nullptr, nullptr, nullptr, Y, 64, nullptr, 0, nullptr),
         OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_gemm_lm(8, 1, P, 0, S, 5, 240, nullptr, W16, 64, nullptr, nullptr, nullptr, Y, 64, nullptr, 0, nullptr),
         OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_gemm_lm(8, 1, P, 0, S, 5, 256, nullptr, W16, 64, S, nullptr, nullptr, Y, 64, nullptr, 0, nullptr),
         OQ_ERR_INVALID_ARG, 0);
  g_stub.fail_next = 1;
  EXPECT(oq_gemm_lm(4, 0, P, 128, S, 5, 256, LV, W16, 64, nullptr, nullptr, nullptr, Y, 64, P, need, nullptr),
         OQ_ERR_HIP, 1);
}

void asym() {
  oq_rot r = rpbh(256, 128, 1);
  uint16_t *H = reinterpret_cast<uint16_t *>(P);
  const float *S = F;
  const uint32_t *U = reinterpret_cast<const uint32_t *>(P);
  EXPECT(oq_quant_weight_asym(F, 64, 256, 256, &r, 64, P, H, H, F, nullptr), OQ_OK, 1);
  EXPECT(oq_quant_weight_asym(F, 64, 96, 96, nullptr, 32, P, H, H, F, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_quant_weight_asym(F, 64, 256, 256, &r, 48, P, H, H, F, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_quant_weight_asym(F, 64, 256, 256, &r, 64, P, reinterpret_cast<uint16_t *>(Q), H, F, nullptr),
         OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_quant_weight_asym(F, 64, 256, 256, &r, 64, P, nullptr, H, F, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_quant_weight_asym(nullptr, 0, 256, 256, &r, 64, nullptr, nullptr, nullptr, nullptr, nullptr), OQ_OK, 0);
  EXPECT(oq_prepack_w4_asym(P, H, H, 64, 256, 64, P, F, reinterpret_cast<uint32_t *>(P), nullptr), OQ_OK, 1);
  EXPECT(oq_prepack_w4_asym(P, H, H, 64, 256, 64, P, F, reinterpret_cast<uint32_t *>(Q4), nullptr), OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_prepack_w4_asym(P, H, H, 64, 256, 128, P, F, reinterpret_cast<uint32_t *>(P), nullptr), OQ_ERR_UNSUPPORTED,
         0);
  uint32_t *G = reinterpret_cast<uint32_t *>(P);
  EXPECT(oq_quant_act_gsum(X, 4, 256, 256, &r, 0, OQ_A4 | OQ_TILED, P, F, G, nullptr, nullptr), OQ_OK, 1);
  EXPECT(oq_quant_act_gsum(X, 4, 256, 256, &r, 1, OQ_A6 | OQ_TILED | OQ_SCALE_PCTL, P, F, G, F, nullptr), OQ_OK, 1);
  EXPECT(oq_quant_act_gsum(X, 4, 256, 256, &r, 0, OQ_A8, P, F, G, nullptr, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_quant_act_gsum(X, 4, 256, 256, &r, 0, OQ_A4 | OQ_TILED, P, F, reinterpret_cast<uint32_t *>(Q), nullptr,
                           nullptr), OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_quant_act_gsum(X, 4, 256, 256, &r, 1, OQ_A4 | OQ_TILED, P, F, G, nullptr, nullptr), OQ_ERR_INVALID_ARG, 0);
  oq_rot r96 = rpbh(96, 32, 1);
  EXPECT(oq_quant_act_gsum(X, 4, 96, 96, &r96, 0, OQ_A4 | OQ_TILED, P, F, G, nullptr, nullptr), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_gemm_w4a4_asym(OQ_A4 | OQ_TILED, P, S, U, 5, 256, P, S, U, 64, nullptr, nullptr, nullptr, Y, 64, nullptr),
         OQ_OK, 1);
  EXPECT(oq_gemm_w4a4_asym(OQ_A6 | OQ_TILED, P, S, U, 5, 256, P, S, U, 64, nullptr, nullptr, nullptr, Y, 64, nullptr),
         OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_gemm_w4a4_asym(OQ_A4 | OQ_TILED, P, S, U, 5, 256, P, S, reinterpret_cast<const uint32_t *>(Q4), 64, nullptr,
                           nullptr, nullptr, Y, 64, nullptr), OQ_ERR_ALIGNMENT, 0);
  EXPECT(oq_gemm_w4a4_asym(OQ_A4 | OQ_TILED, P, S, nullptr, 5, 256, P, S, U, 64, nullptr, nullptr, nullptr, Y, 64,
                           nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_gemm_w4a4_asym(OQ_A4 | OQ_TILED, P, S, U, 400000, 16384, P, S, U, 64, nullptr, nullptr, nullptr, Y, 64,
                           nullptr), OQ_ERR_UNSUPPORTED, 0);
}

void kron_plan_probe() {
  int32_t m = 0, b = 0, np = 0;
  EXPECT(oq_kron_plan(0, &m, &b, &np), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_kron_plan(20000, &m, &b, &np), OQ_ERR_UNSUPPORTED, 0);
  EXPECT(oq_kron_plan(3072, nullptr, &b, &np), OQ_ERR_INVALID_ARG, 0);
  // the plan is the smallest m * b >= n over m in {1, 12, 36, 44} and powers of two b >= 16
  bool all = true;
  for (int n = 1; n <= 16384; n += 97) {
    if (oq_kron_plan(n, &m, &b, &np) != OQ_OK) {
      all = false;
      break;
    }
    int best = 1 << 30;
    for (int mm : {1, 12, 36, 44})
      for (int bb = 16; bb <= 16384; bb *= 2)
        if (mm * bb >= n && mm * bb <= 16384 && mm * bb < best) best = mm * bb;
    all = all && np == m * b && np == best && (b & (b - 1)) == 0 && b >= 16;
  }
  TRUE(all);

  float *sink = F;
  double ops = 0.0;
  EXPECT(oq_probe_mfma(OQ_PROBE_FP6, 10, sink, &ops, nullptr), OQ_OK, 1);
  EXPECT(oq_probe_mfma(0, 10, sink, &ops, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_probe_mfma(OQ_PROBE_FP6_UPDATE, 10, sink, &ops, nullptr), OQ_OK, 1);
  EXPECT(oq_probe_mfma(8, 10, sink, &ops, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_probe_mfma(OQ_PROBE_F16, 0, sink, &ops, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_probe_mfma(OQ_PROBE_F16, (1 << 20) + 1, sink, &ops, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_probe_mfma(OQ_PROBE_F16, 10, nullptr, &ops, nullptr), OQ_ERR_INVALID_ARG, 0);
  EXPECT(oq_probe_mfma(OQ_PROBE_F16, 10, sink, nullptr, nullptr), OQ_ERR_INVALID_ARG, 0);
  TRUE(oq_probe_sink_elems() == 512u * 256u);
}

}  // namespace

int main() {
  for (int i = 0; i < 8; ++i) {
    g_perm[i] = i;
    g_signs[i] = 1;
  }
  reset();
  center_rotate();
  quant_act();
  quant_weight_prepack();
  gemms();
  fused();
  lloyd_max();
  asym();
  kron_plan_probe();
  if (g_fail) {
    std::printf("%d of %d cases failed\n", g_fail, g_cases);
    return 1;
  }
  std::printf("%d cases passed\n", g_cases);
  return 0;
}
