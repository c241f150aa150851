// K5: MXFP4 activations x MXFP4 weights on the gfx950 scaled FP4 MFMA.
//
// y[t][o] = bf16( sum_blocks 2^(ea + ew) sum_{k in block} fp4(a) fp4(w) + bias[o] )
// (WUSH review, "Core claim" and Fig. 2 caption: MXFP4 block quantizers with
// G = 32; the element and scale formats are those of the OCP MX v1.0
// specification the review cites.)
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in E2M1: lane l holds
// row l%32 and the 32 consecutive k of half l/32 as 16 bytes with element j
// in bits 4j..4j+3, which is exactly the row-major two-codes-per-byte layout
// of the codes, and its E8M0 byte scales those 32 elements.  So operands are
// loaded straight from the code rows; the accumulator carries the whole K.
#include "oq_internal.h"

#include <atomic>
#include <type_traits>

namespace oq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256)
gemm_mx_kernel(const uint8_t *__restrict__ qa, int64_t lda, const uint8_t *__restrict__ ea, int64_t M,
               int K, const uint8_t *__restrict__ w, const uint8_t *__restrict__ ew, int N,
               const float *__restrict__ bias, uint16_t *__restrict__ y, int64_t ldy) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t m0 = (int64_t)blockIdx.y * 128 + (wave >> 1) * 64;
  const int n0 = blockIdx.x * 128 + (wave & 1) * 64;
  const int r32 = lane & 31;
  const int half = lane >> 5;
  const int KB = K / 32;

  int64_t arow[2];
  bool aok[2];
  int wrow[2];
  bool wok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    arow[i] = m0 + 32 * i + r32;
    aok[i] = arow[i] < M;
    wrow[i] = n0 + 32 * i + r32;
    wok[i] = wrow[i] < N;
  }
  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (v16f){};

  for (int k0 = 0; k0 < K; k0 += 64) {
    const int kb = k0 / 32 + half;
    v8i A[2], B[2];
    int sa[2], sb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 p = aok[i] ? *reinterpret_cast<const uint4 *>(qa + arow[i] * lda + kb * 16) : make_uint4(0u, 0u, 0u, 0u);
      A[i] = (v8i){(int)p.x, (int)p.y, (int)p.z, (int)p.w, 0, 0, 0, 0};
      sa[i] = aok[i] ? (int)ea[arow[i] * KB + kb] : 127;
      const uint4 q = wok[i] ? *reinterpret_cast<const uint4 *>(w + (int64_t)wrow[i] * (K / 2) + kb * 16) : make_uint4(0u, 0u, 0u, 0u);
      B[i] = (v8i){(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
      sb[i] = wok[i] ? (int)ew[(int64_t)wrow[i] * KB + kb] : 127;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[i], B[j], acc[i][j], 4, 4, 0, sa[i], 0, sb[j]);
  }

#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = m0 + 32 * i + (r >> 2) * 8 + half * 4 + (r & 3);
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + 32 * j + r32;
        if (col >= N) continue;
        float v = acc[i][j][r];
        if (bias) v = v + bias[col];
        y[row * ldy + col] = f32_to_bf16_rne(v);
      }
    }
  }
}


typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt vmcnt(C) (and lgkmcnt(0)): the fields of the gfx9 encoding
template <int C>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(0x0F70 | (C & 0xF) | ((C >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Global -> LDS copies from a wave-uniform base (SGPRs) plus a 32-bit lane
// offset: each lane moves 16 (or 4) bytes to lds_addr + lane * 16 (or * 4).
// Inline asm for the reason given at dma_lds16; no register outputs.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_s(const void *sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_s(const void *sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Tiled variant: WM x WN wavefronts, each owning TM x TN MFMA tiles of 32 x 32
// (accumulators carry the whole K).  Each stage holds 128 k (two MFMA k-steps):
//   A: (BM/32) row blocks x 2 k-halves of 1 KiB, laid out so lane l of the
//      fragment finds its 16 bytes at offset 16 l (row l % 32, k-half l / 32);
//   B: the same for the weight rows;
//   SA, SB: one 32-bit word per row = the four E8M0 bytes of the stage's 128 k.
// All of it is copied global -> LDS with global_load_lds (16-byte units for
// codes, 4-byte units for scales) into an NSTAGE ring, one barrier per stage.
template <int WM, int WN, int TM, int TN, int NSTAGE>
struct MxCfg {
  static constexpr int WAVES = WM * WN;
  static constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  static constexpr int A_BYTES = (BM / 32) * 2 * 1024, B_BYTES = (BN / 32) * 2 * 1024;
  static constexpr int SA_BYTES = BM * 4, SB_BYTES = BN * 4;
  static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
  static constexpr int U16 = (A_BYTES + B_BYTES) / 1024;  // 16-byte-per-lane units
  static constexpr int U4 = (SA_BYTES + SB_BYTES) / 256;  // 4-byte-per-lane units
  static constexpr int P16 = U16 / WAVES, P4 = (U4 + WAVES - 1) / WAVES;
  static_assert(U16 % WAVES == 0, "code units must divide evenly among the waves");
  static_assert(NSTAGE >= 2 && NSTAGE <= 4, "ring depth");
};

// Row-major codes and E8M0 bytes (the boundary layout): each copy unit
// gathers 32 rows.  Tiled operands take the prefetching kernel below.
template <int WM, int WN, int TM, int TN, int NSTAGE>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_mx_tiled_kernel(const uint8_t *__restrict__ qa, int64_t lda, const uint8_t *__restrict__ ea, int64_t M, int K,
                     const uint8_t *__restrict__ w, const uint8_t *__restrict__ ew, int N,
                     const float *__restrict__ bias, uint16_t *__restrict__ y, int64_t ldy) {
  using C = MxCfg<WM, WN, TM, TN, NSTAGE>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KB = K / 32;
  const int S = K / 128;  // stages
  const int64_t m0 = (int64_t)blockIdx.y * C::BM;
  const int n0 = blockIdx.x * C::BN;

  // ---- per-lane DMA sources (stage 0) and LDS offsets of this wave's units
  const uint8_t *src16[C::P16];
  int off16[C::P16];
#pragma unroll
  for (int q = 0; q < C::P16; ++q) {
    const int u = wave + q * C::WAVES;
    const int r = lane & 31, hf = lane >> 5;
    if (u < C::A_BYTES / 1024) {
      const int blk = u >> 1, kk = u & 1;
      int64_t row = m0 + 32 * blk + r;
      if (row > M - 1) row = M - 1;
      src16[q] = qa + row * lda + 32 * kk + 16 * hf;
    } else {
      const int v = u - C::A_BYTES / 1024;
      const int blk = v >> 1, kk = v & 1;
      int row = n0 + 32 * blk + r;
      if (row > N - 1) row = N - 1;
      src16[q] = w + (int64_t)row * (K / 2) + 32 * kk + 16 * hf;
    }
    off16[q] = u * 1024;
  }
  const uint8_t *src4[C::P4];
  int off4[C::P4];
  int64_t inc4[C::P4];
#pragma unroll
  for (int q = 0; q < C::P4; ++q) {
    const int u = wave + q * C::WAVES;
    off4[q] = -1;
    src4[q] = ea;
    inc4[q] = 4;
    if (u < C::SA_BYTES / 256) {
      int64_t row = m0 + 64 * u + lane;
      if (row > M - 1) row = M - 1;
      src4[q] = ea + row * KB;
      inc4[q] = 4;
      off4[q] = C::A_BYTES + C::B_BYTES + u * 256;
    } else if (u < C::U4) {
      const int v = u - C::SA_BYTES / 256;
      int row = n0 + 64 * v + lane;
      if (row > N - 1) row = N - 1;
      src4[q] = ew + (int64_t)row * KB;
      inc4[q] = 4;
      off4[q] = C::A_BYTES + C::B_BYTES + C::SA_BYTES + v * 256;
    }
  }
  const int64_t inc16 = 64;  // bytes of codes per stage of 128 k
  // number of DMA instructions this wave issues per stage
  const int n4 = (C::U4 - wave + C::WAVES - 1) / C::WAVES;
  const int per_stage = C::P16 + n4;

  // One static LDS array per ring slot and the k loop unrolled by the ring
  // depth, so that every slot reference is a compile-time choice of array:
  // the compiler can then tell that copies in flight into the other slots do
  // not alias this slot's reads, and waits only for the copies of this slot.
  __shared__ __attribute__((aligned(16))) uint8_t ring0[C::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[C::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[NSTAGE > 2 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t ring3[NSTAGE > 3 ? C::STAGE : 16];
  auto slot = [&](auto jc) -> uint8_t * {
    constexpr int j = decltype(jc)::value;
    if constexpr (j == 0) return ring0;
    else if constexpr (j == 1) return ring1;
    else if constexpr (j == 2) return ring2;
    else return ring3;
  };
  auto issue = [&](auto jc, int ks) {
    const uint32_t base = lds_addr_of(slot(jc));
#pragma unroll
    for (int q = 0; q < C::P16; ++q) dma_lds16(src16[q] + (int64_t)ks * inc16, base + off16[q]);
#pragma unroll
    for (int q = 0; q < C::P4; ++q)
      if (off4[q] >= 0) dma_lds4(src4[q] + (int64_t)ks * inc4[q], base + off4[q]);
  };

  const int wm = wave / WN, wn = wave % WN;
  const int r = lane & 31, hf = lane >> 5;
  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (v16f){};

  if (0 < S) issue(std::integral_constant<int, 0>{}, 0);
  if (1 < S) issue(std::integral_constant<int, 1>{}, 1);
  if constexpr (NSTAGE > 3)
    if (2 < S) issue(std::integral_constant<int, 2>{}, 2);

  // one stage: slot J holds k-slice ks
  auto body = [&](auto jc, int ks) {
    constexpr int J = decltype(jc)::value;
    // this wave's copies of slot J are done once at most the copies of the
    // stages issued after it are outstanding; the barrier then publishes
    // every wave's copies of slot J
    const int ahead = min(NSTAGE - 2, S - 1 - ks);
    if (ahead == NSTAGE - 2 && per_stage == C::P16 + C::P4)
      wait_vm<(NSTAGE - 2) * (C::P16 + C::P4)>();
    else if (ahead == NSTAGE - 2)
      wait_vm<(NSTAGE - 2) * (C::P16 + C::P4 - 1)>();
    else
      wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    // refill the slot consumed at ks - 1 (every wave is past it)
    if (ks + NSTAGE - 1 < S) issue(std::integral_constant<int, (J + NSTAGE - 1) % NSTAGE>{}, ks + NSTAGE - 1);

    const uint8_t *stage = slot(jc);
    const uint32_t *sA = reinterpret_cast<const uint32_t *>(stage + C::A_BYTES + C::B_BYTES);
    const uint32_t *sB = sA + C::BM;
    uint32_t wa[TM], wb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) wa[i] = sA[wm * 32 * TM + 32 * i + r];
#pragma unroll
    for (int j = 0; j < TN; ++j) wb[j] = sB[wn * 32 * TN + 32 * j + r];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      v8i A[TM], B[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const uint4 p = *reinterpret_cast<const uint4 *>(stage + ((wm * TM + i) * 2 + kk) * 1024 + 16 * lane);
        A[i] = (v8i){(int)p.x, (int)p.y, (int)p.z, (int)p.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint4 p = *reinterpret_cast<const uint4 *>(stage + C::A_BYTES + ((wn * TN + j) * 2 + kk) * 1024 + 16 * lane);
        B[j] = (v8i){(int)p.x, (int)p.y, (int)p.z, (int)p.w, 0, 0, 0, 0};
      }
      const int sh = 8 * (2 * kk + hf);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[i], B[j], acc[i][j], 4, 4, 0,
                                                                      (int)((wa[i] >> sh) & 0xFF), 0,
                                                                      (int)((wb[j] >> sh) & 0xFF));
    }
  };

  for (int ks = 0; ks < S; ks += NSTAGE) {
    body(std::integral_constant<int, 0>{}, ks);
    if (ks + 1 < S) body(std::integral_constant<int, 1>{}, ks + 1);
    if constexpr (NSTAGE > 2)
      if (ks + 2 < S) body(std::integral_constant<int, 2>{}, ks + 2);
    if constexpr (NSTAGE > 3)
      if (ks + 3 < S) body(std::integral_constant<int, 3>{}, ks + 3);
  }

  // ---- epilogue: + bias, bf16, staged per 32-row slab in LDS for 16-byte stores
  float bv[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n0 + wn * 32 * TN + 32 * j + r;
    bv[j] = (bias && col < N) ? bias[col] : 0.f;
  }
  __syncthreads();  // every wave is done with the ring
  constexpr int SROW = 64 * TN + 16;  // bytes per staged row (32 TN bf16 + pad)
  constexpr int PER_SLOT = C::STAGE / (32 * SROW);  // staging areas per ring slot
  static_assert(PER_SLOT * NSTAGE >= C::WAVES, "epilogue staging must fit in the ring");
  const int sw = wave / PER_SLOT, so = (wave % PER_SLOT) * (32 * SROW);
  uint8_t *stg = (sw == 0 ? ring0 : sw == 1 ? ring1 : sw == 2 ? ring2 : ring3) + so;
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(y) & 15) == 0) && (ldy % 8 == 0);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int rr = (e >> 2) * 8 + hf * 4 + (e & 3);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        float v = acc[i][j][e];
        if (bias) v = v + bv[j];
        *reinterpret_cast<uint16_t *>(stg + rr * SROW + (32 * j + r) * 2) = f32_to_bf16_rne(v);
      }
    }
    // 16 bytes per lane: 4 TN lanes cover one staged row
    constexpr int LPR = 4 * TN, RPP = 64 / LPR;
    const int cl = (lane % LPR) * 8;
    const int col = n0 + wn * 32 * TN + cl;
#pragma unroll
    for (int q = 0; q < 32 / RPP; ++q) {
      const int rr = lane / LPR + RPP * q;
      const int64_t row = m0 + wm * 32 * TM + 32 * i + rr;
      const uint4 v = *reinterpret_cast<const uint4 *>(stg + rr * SROW + cl * 2);
      if (row >= M) continue;
      uint16_t *dst = y + row * ldy + col;
      if (vec_ok && col + 8 <= N) {
        *reinterpret_cast<uint4 *>(dst) = v;
      } else {
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int c = 0; c < 8; ++c)
          if (col + c < N) dst[c] = (uint16_t)(wv[c >> 1] >> (16 * (c & 1)));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Prefetching kernel for tiled operands.  Workgroups of WM x WN wavefronts,
// each owning TM x TN MFMA tiles of 32 x 32 (accumulators carry the whole
// K).  A stage is one 128-wide k-slice (two MFMA k-steps) in a ring of four
// LDS slots:
//   A: (BM/32) row blocks x 2 k-groups of 1 KiB (row block b, k-group h at
//      (2b + h) KiB; the two tiles are adjacent in the tiled layout);
//   B: the same for the weight rows;
//   SA, SB: the slice's scale word of each row.
// Each wave copies P16 1-KiB units (16 bytes a lane) and one 256-byte unit of
// scale words per stage with global_load_lds, from a wave-uniform base plus
// a loop-invariant lane offset.  One barrier per slice:
//   top of slice s: own copies of slice s+1 done (only those of slices s+2
//   and s+3 may be outstanding) and own LDS reads done -> barrier -> copy
//   slice s+4 into the slot of slice s, whose fragments are already in
//   registers;
//   during slice s: each fragment register is reloaded with slice s+1 right
//   after the last MFMA of slice s that reads it, the scale words at the
//   start of the slice.
// So every slice starts with its operands in registers, and a copy has three
// slices of compute to land.
// REMAP: the linear workgroup id is assumed to go round-robin over the 8 XCDs
// (as the dispatcher hands them out); each XCD is given one contiguous run of
// output tiles, walked GROUP_M row blocks at a time, so the workgroups that
// share an L2 at any moment cover a compact block of A rows and B columns.
// ---------------------------------------------------------------------------
template <int WM, int WN, int TM, int TN>
struct MxP {
  static constexpr int WAVES = WM * WN, NSLOT = 4;
  static constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  static constexpr int A_BYTES = (BM / 32) * 2048, B_BYTES = (BN / 32) * 2048;
  static constexpr int SA_BYTES = BM * 4, SB_BYTES = BN * 4;
  static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
  static constexpr int P16 = (A_BYTES + B_BYTES) / 1024 / WAVES;
  static constexpr int P4 = (SA_BYTES + SB_BYTES) / 256 / WAVES;
  static constexpr int PER_STAGE = P16 + P4;  // copy instructions per wave per stage
  static constexpr int OCC = WAVES >= 8 ? 2 : 1;  // waves per SIMD (one workgroup per CU)
  static constexpr int SROW = 64 * TN + 16;  // padded bytes per staged output row
  static constexpr int LDS_BYTES = NSLOT * STAGE;
  static constexpr int GROUP_M = 8;
  static_assert((A_BYTES + B_BYTES) % (1024 * WAVES) == 0, "code units divide evenly among the waves");
  static_assert((SA_BYTES + SB_BYTES) % (256 * WAVES) == 0 && SA_BYTES % 256 == 0, "scale units divide evenly");
  static_assert(2 * PER_STAGE <= 63, "vmcnt range");
  static_assert(WAVES * 32 * SROW <= LDS_BYTES, "epilogue staging fits in the ring");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <int WM, int WN, int TM, int TN, bool REMAP>
__global__ void __launch_bounds__(64 * WM * WN)
__attribute__((amdgpu_waves_per_eu(MxP<WM, WN, TM, TN>::OCC, MxP<WM, WN, TM, TN>::OCC)))
gemm_mx_pf_kernel(const uint8_t *__restrict__ qa, const uint8_t *__restrict__ ea, int64_t M, int K,
                  const uint8_t *__restrict__ w, const uint8_t *__restrict__ ew, int N,
                  const float *__restrict__ bias, uint16_t *__restrict__ y, int64_t ldy) {
  using C = MxP<WM, WN, TM, TN>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const uint32_t lds0 = lds_addr_of(smem);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = K / 128;  // k-slices
  const int G = K / 64;
  const int64_t Mp = (M + 31) / 32 * 32;
  const int Np = (N + 31) / 32 * 32;

  int tm = blockIdx.y, tn = blockIdx.x;
  if constexpr (REMAP) {
    const int gx = gridDim.x, gy = gridDim.y, T = gx * gy;
    const int lid = blockIdx.x + blockIdx.y * gx;
    const int xcd = lid % 8, idx = lid / 8, q = T / 8, rr = T % 8;
    const int t = xcd * q + (xcd < rr ? xcd : rr) + idx;  // XCD c owns tiles [c q + min(c, rr), ...)
    const int grp = t / (C::GROUP_M * gx), g0 = grp * C::GROUP_M;
    const int rows = gy - g0 < C::GROUP_M ? gy - g0 : C::GROUP_M;
    const int within = t - grp * C::GROUP_M * gx;
    tm = g0 + within % rows;
    tn = within / rows;
  }
  const int64_t m0 = (int64_t)tm * C::BM;
  const int n0 = tn * C::BN;

  // ---- copy units of this wave: uniform base (slice 0) + lane offset
  const uint8_t *cbase[C::P16];
  uint32_t clds[C::P16];
#pragma unroll
  for (int q = 0; q < C::P16; ++q) {
    const int u = wave + q * C::WAVES;
    if (u < C::A_BYTES / 1024) {
      int64_t rb = m0 / 32 + u / 2;
      if (rb > Mp / 32 - 1) rb = Mp / 32 - 1;
      cbase[q] = qa + (rb * G + (u & 1)) * 1024;
    } else {
      const int v = u - C::A_BYTES / 1024;
      int cb = n0 / 32 + v / 2;
      if (cb > Np / 32 - 1) cb = Np / 32 - 1;
      cbase[q] = w + ((int64_t)cb * G + (v & 1)) * 1024;
    }
    clds[q] = 1024u * u;
  }
  // scale words: unit u covers rows row0 + lane of A (u below BM / 64) or of
  // B, clamped to the padded extent; slice s adds s * Mp (or Np) words
  const uint8_t *sbase[C::P4];
  int64_t sstep[C::P4];
  uint32_t soff[C::P4], slds[C::P4];
#pragma unroll
  for (int q = 0; q < C::P4; ++q) {
    const int u = wave + q * C::WAVES;
    if (u < C::BM / 64) {
      int64_t row0 = m0 + 64 * u;
      if (row0 > Mp - 1) row0 = Mp - 1;
      const int64_t rl = row0 + lane > Mp - 1 ? Mp - 1 : row0 + lane;
      sbase[q] = ea + row0 * 4;
      sstep[q] = Mp * 4;
      soff[q] = (uint32_t)(4 * (rl - row0));
      slds[q] = C::A_BYTES + C::B_BYTES + 256u * u;
    } else {
      const int v = u - C::BM / 64;
      int row0 = n0 + 64 * v;
      if (row0 > Np - 1) row0 = Np - 1;
      const int rl = row0 + lane > Np - 1 ? Np - 1 : row0 + lane;
      sbase[q] = ew + (int64_t)row0 * 4;
      sstep[q] = (int64_t)Np * 4;
      soff[q] = (uint32_t)(4 * (rl - row0));
      slds[q] = C::A_BYTES + C::B_BYTES + C::SA_BYTES + 256u * v;
    }
  }
  const uint32_t loff = 16u * lane;

  auto issue = [&](int slot, int s) {
    const uint32_t base = lds0 + slot * C::STAGE;
#pragma unroll
    for (int q = 0; q < C::P16; ++q) dma16_s(cbase[q] + (int64_t)s * 2048, loff, base + clds[q]);
#pragma unroll
    for (int q = 0; q < C::P4; ++q) dma4_s(sbase[q] + (int64_t)s * sstep[q], soff[q], base + slds[q]);
  };

  const int wm = wave / WN, wn = wave % WN;
  const int r = lane & 31, hf = lane >> 5;
  const uint8_t *fa = smem + (wm * TM) * 2048 + 16 * lane;
  const uint8_t *fb = smem + C::A_BYTES + (wn * TN) * 2048 + 16 * lane;
  // E8M0 byte of row r, k-step kk and lane half hf: byte 2 kk + hf of the
  // row's scale word, read on its own (no VALU extraction)
  const uint8_t *fsa = smem + C::A_BYTES + C::B_BYTES + 4 * (wm * 32 * TM + r) + hf;
  const uint8_t *fsb = smem + C::A_BYTES + C::B_BYTES + C::SA_BYTES + 4 * (wn * 32 * TN + r) + hf;

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (v16f){};

  auto frag = [](const uint8_t *p) {
    const uint4 v = *reinterpret_cast<const uint4 *>(p);
    return (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  };

  // ---- prologue: slices 0..3 in flight, slice 0 complete, its operands loaded
#pragma unroll
  for (int p = 0; p < C::NSLOT; ++p)
    if (p < S) issue(p, p);
  if (S > 3) wait_vm<3 * C::PER_STAGE>();
  else if (S > 2) wait_vm<2 * C::PER_STAGE>();
  else if (S > 1) wait_vm<C::PER_STAGE>();
  else wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  v8i A[2][TM], B[2][TN];
  int sa[2][TM], sb[2][TN], nsa[2][TM], nsb[2][TN];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int i = 0; i < TM; ++i) A[kk][i] = frag(fa + i * 2048 + kk * 1024);
#pragma unroll
    for (int j = 0; j < TN; ++j) B[kk][j] = frag(fb + j * 2048 + kk * 1024);
#pragma unroll
    for (int i = 0; i < TM; ++i) sa[kk][i] = fsa[128 * i + 2 * kk];
#pragma unroll
    for (int j = 0; j < TN; ++j) sb[kk][j] = fsb[128 * j + 2 * kk];
  }

  // one slice from registers; slice s+1's operands (slot JN) reloaded into
  // each register after its last use.  Tiles run column-major when TM > TN,
  // so a reloaded A fragment is next needed TN tiles... one slice later.
  auto slice = [&](auto jnc) {
    constexpr int JN = decltype(jnc)::value;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < TM; ++i) nsa[kk][i] = fsa[JN * C::STAGE + 128 * i + 2 * kk];
#pragma unroll
      for (int j = 0; j < TN; ++j) nsb[kk][j] = fsb[JN * C::STAGE + 128 * j + 2 * kk];
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int t = 0; t < TM * TN; ++t) {
        const int i = TM >= TN ? t % TM : t / TN, j = TM >= TN ? t / TM : t % TN;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[kk][i], B[kk][j], acc[i][j], 4, 4, 0,
                                                                    sa[kk][i], 0, sb[kk][j]);
        __builtin_amdgcn_sched_barrier(0);
        if (j == TN - 1) A[kk][i] = frag(fa + JN * C::STAGE + i * 2048 + kk * 1024);
        if (i == TM - 1) B[kk][j] = frag(fb + JN * C::STAGE + j * 2048 + kk * 1024);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < TM; ++i) sa[kk][i] = nsa[kk][i];
#pragma unroll
      for (int j = 0; j < TN; ++j) sb[kk][j] = nsb[kk][j];
    }
  };

  auto body = [&](auto jc, int s) {
    constexpr int J = decltype(jc)::value;  // s % 4
    if (s + 3 < S) wait_vm<2 * C::PER_STAGE>();
    else if (s + 2 < S) wait_vm<C::PER_STAGE>();
    else wait_vm<0>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    if (s + 4 < S) issue(J, s + 4);
    __builtin_amdgcn_sched_barrier(0);
    slice(std::integral_constant<int, (J + 1) % 4>{});
  };
  for (int s = 0; s < S; s += 4) {
    body(std::integral_constant<int, 0>{}, s);
    if (s + 1 < S) body(std::integral_constant<int, 1>{}, s + 1);
    if (s + 2 < S) body(std::integral_constant<int, 2>{}, s + 2);
    if (s + 3 < S) body(std::integral_constant<int, 3>{}, s + 3);
  }

  // ---- epilogue: + bias, bf16, staged per 32-row slab in LDS for 16-byte stores
  float bv[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n0 + wn * 32 * TN + 32 * j + r;
    bv[j] = (bias && col < N) ? bias[col] : 0.f;
  }
  wait_vm<0>();
  __syncthreads();  // every wave is done with the ring
  uint8_t *stg = smem + wave * (32 * C::SROW);
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(y) & 15) == 0) && (ldy % 8 == 0);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int rr = (e >> 2) * 8 + hf * 4 + (e & 3);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        float v = acc[i][j][e];
        if (bias) v = v + bv[j];
        *reinterpret_cast<uint16_t *>(stg + rr * C::SROW + (32 * j + r) * 2) = f32_to_bf16_rne(v);
      }
    }
    // 16 bytes per lane: 4 TN lanes cover one staged row
    constexpr int LPR = 4 * TN, RPP = 64 / LPR;
    const int cl = (lane % LPR) * 8;
    const int col = n0 + wn * 32 * TN + cl;
#pragma unroll
    for (int q = 0; q < 32 / RPP; ++q) {
      const int rr = lane / LPR + RPP * q;
      const int64_t row = m0 + wm * 32 * TM + 32 * i + rr;
      const uint4 v = *reinterpret_cast<const uint4 *>(stg + rr * C::SROW + cl * 2);
      if (row >= M) continue;
      uint16_t *dst = y + row * ldy + col;
      if (vec_ok && col + 8 <= N) {
        *reinterpret_cast<uint4 *>(dst) = v;
      } else {
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int c = 0; c < 8; ++c)
          if (col + c < N) dst[c] = (uint16_t)(wv[c >> 1] >> (16 * (c & 1)));
      }
    }
  }
}

template <int WM, int WN, int TM, int TN, bool REMAP>
hipError_t launch_mx_pf(const uint8_t *qa, const uint8_t *ea, int64_t M, int K, const uint8_t *w, const uint8_t *ew,
                        int N, const float *bias, uint16_t *y, int64_t ldy, hipStream_t stream) {
  using C = MxP<WM, WN, TM, TN>;
  auto kern = gemm_mx_pf_kernel<WM, WN, TM, TN, REMAP>;
  static std::atomic<bool> attr_set[64];
  const hipError_t e = lds_limit_once((const void *)kern, C::LDS_BYTES, attr_set);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((N + C::BN - 1) / C::BN), (unsigned)((M + C::BM - 1) / C::BM));
  hipLaunchKernelGGL(kern, grid, dim3(64 * C::WAVES), C::LDS_BYTES, stream, qa, ea, M, K, w, ew, N, bias, y, ldy);
  return hipGetLastError();
}

template <int WM, int WN, int TM, int TN, int NSTAGE>
hipError_t launch_mx_staged(const uint8_t *qa, int64_t lda, const uint8_t *ea, int64_t M, int K, const uint8_t *w,
                            const uint8_t *ew, int N, const float *bias, uint16_t *y, int64_t ldy,
                            hipStream_t stream) {
  using C = MxCfg<WM, WN, TM, TN, NSTAGE>;
  dim3 grid((unsigned)((N + C::BN - 1) / C::BN), (unsigned)((M + C::BM - 1) / C::BM));
  hipLaunchKernelGGL((gemm_mx_tiled_kernel<WM, WN, TM, TN, NSTAGE>), grid, dim3(64 * C::WAVES), 0, stream, qa, lda,
                     ea, M, K, w, ew, N, bias, y, ldy);
  return hipGetLastError();
}

// canonical MXFP4 weights (codes [N][K/2], E8M0 [N][K/32]) -> tiled layout:
// one thread per (row < Np, k-group, half): 16 code bytes, plus the four scale
// bytes of a 128-wide k-slice from the thread of its first k-group and half 0.
// Rows N..Np-1 get zero codes and unit scales.
__global__ void prepack_mx_kernel(const uint8_t *__restrict__ w, const uint8_t *__restrict__ ew, int N, int Np, int K,
                                  uint8_t *__restrict__ out, uint8_t *__restrict__ out_s) {
  const int G = K / 64;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)Np * G * 2) return;
  const int half = (int)(idx & 1);
  const int64_t rg = idx >> 1;
  const int kg = (int)(rg % G);
  const int row = (int)(rg / G);
  uint4 c = make_uint4(0u, 0u, 0u, 0u);
  if (row < N) c = *reinterpret_cast<const uint4 *>(w + (int64_t)row * (K / 2) + kg * 32 + half * 16);
  *reinterpret_cast<uint4 *>(out + ((int64_t)(row / 32) * G + kg) * 1024 + 16 * (32 * half + row % 32)) = c;
  if (half == 0 && (kg & 1) == 0) {
    uint32_t sw = 0x7F7F7F7Fu;
    if (row < N) {
      const uint8_t *sp = ew + (int64_t)row * (K / 32) + 2 * kg;
      sw = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8) | ((uint32_t)sp[2] << 16) | ((uint32_t)sp[3] << 24);
    }
    *reinterpret_cast<uint32_t *>(out_s + ((int64_t)(kg / 2) * Np + row) * 4) = sw;
  }
}

}  // namespace

hipError_t launch_gemm_mx(int tiled_in, const uint8_t *qa, int64_t lda_bytes, const uint8_t *a_e8m0, int64_t M,
                          int K, const uint8_t *w, const uint8_t *w_e8m0, int N, const float *bias, uint16_t *y,
                          int64_t ldy, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  // tiled operands: the prefetching kernel, 8 waves of 128 x 64 outputs per
  // 256 x 256 workgroup tile, XCD-grouped tile order
  if (tiled_in) return launch_mx_pf<2, 4, 4, 2, true>(qa, a_e8m0, M, K, w, w_e8m0, N, bias, y, ldy, stream);
  // row-major operands: the staged kernel copies the four E8M0 bytes of a
  // 128-wide k-slice as one 32-bit word and the codes in 16-byte pieces
  const bool staged = K % 128 == 0 && lda_bytes % 16 == 0 &&
                      ((reinterpret_cast<uintptr_t>(qa) | reinterpret_cast<uintptr_t>(w)) & 15) == 0 &&
                      ((reinterpret_cast<uintptr_t>(a_e8m0) | reinterpret_cast<uintptr_t>(w_e8m0)) & 3) == 0;
  if (staged)
    return launch_mx_staged<2, 4, 4, 2, 3>(qa, lda_bytes, a_e8m0, M, K, w, w_e8m0, N, bias, y, ldy, stream);
  dim3 grid((unsigned)((N + 127) / 128), (unsigned)((M + 127) / 128));
  hipLaunchKernelGGL(gemm_mx_kernel, grid, dim3(256), 0, stream, qa, lda_bytes, a_e8m0, M, K, w, w_e8m0, N,
                     bias, y, ldy);
  return hipGetLastError();
}

hipError_t launch_prepack_mx(const uint8_t *w, const uint8_t *w_e8m0, int N, int K, uint8_t *out, uint8_t *out_s,
                             hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int Np = (N + 31) / 32 * 32;
  const int64_t total = (int64_t)Np * (K / 64) * 2;
  hipLaunchKernelGGL(prepack_mx_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, w, w_e8m0, N, Np,
                     K, out, out_s);
  return hipGetLastError();
}

}  // namespace oq
