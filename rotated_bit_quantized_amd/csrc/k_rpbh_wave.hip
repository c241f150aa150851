// K1 (activation path): per-token (center) -> RPBH rounds -> absmax quantize
// -> pack, one wavefront per token row, gfx950.
//
// Same arithmetic as the workgroup kernel in k_rpbh.hip (CentriQ Sec. 4.2
// Eq. 4 centering; OrbitQuant PR #25 RPBH rounds; CentriQ Sec. 3 Eq. 1
// absmax codes), organised so that the row loop has no workgroup barrier:
//   * lane l owns, for each 1024-wide slot s of the row, the 16 consecutive
//     coordinates 1024 s + 16 l + j (j = 0..15);
//   * each wave keeps its row in LDS twice, as +x and -x; the gather offset
//     of output i points into the copy whose sign is s_r[i], so the gather
//     applies the sign.  The offsets of every round live in a workgroup LDS
//     table written once, read per row with 16-byte loads.  With one round
//     the row is kept once, each coordinate's sign applied as it is written
//     (a sign mask scattered through the permutation; centring adds the same
//     mask into the sign of m), and 8-wave workgroups run 4 waves per SIMD
//     (4-wave ones at 3 per SIMD when centring);
//   * the first round gathers bfloat16 copies (the loaded words and their
//     sign-flipped twins, no conversion on the write side); centering
//     subtracts s_i m after the gather, which equals s_i RN32(x - m);
//     a second round gathers float32 copies of the first round's outputs;
//   * butterfly stages of stride 1..8 run in registers; strides 16..h/2
//     pair lanes.  Those stages keep each value up to a per-lane sign:
//     every lane adds c times its partner's value (c = -1 on the lane whose
//     index bit is set), which yields a + b on the low lane and -(a - b) on
//     the high lane, each rounded once; the sign the high lanes pick up is a
//     fixed pattern, applied when the values are used.  As an accumulate of
//     a DPP operand this is one v_fmac_f32_dpp per value for lane distances
//     1, 2 (quad_perm), and for the half-row and row mirrors, which pair
//     lane l with l ^ 7 and l ^ 15: lanes are renumbered so that those
//     pairings flip exactly one index bit (index_lane below).  Distances 16
//     and 32 stay in the VALU too: v_permlane16_swap / v_permlane32_swap
//     exchange row or half-wave pieces of two values so that every lane
//     holds both operands of one butterfly, the lane forms a + b and a - b
//     (true signs: both partners carry the same lane sign), and a second
//     swap puts the results back;
//   * when h is a power of 4, 1/sqrt(h) is a power of two: the per-round
//     multiply is exact and is deferred into the quantization scale
//     (identical codes and scales; the float32 output mode applies it);
//   * the row range (absmax) is a wavefront reduction; with the percentile
//     range (CentriQ Sec. 4.2 "Scale and grid") each lane keeps its four
//     largest magnitudes and the wavefront merges those lists, which gives the
//     order statistics the interpolated 0.9995-quantile needs for d <= 4096;
//   * the factorised rotation (H_m (x) H_b) / sqrt(n') of CentriQ Sec. 4.2
//     "Rotation" / App. B.1 (template KM = m; m = 1 is the Sylvester
//     transform of the whole row, up to 4096 wide): lanes load the index-lane
//     chunks of the row directly (centred over the native width, zero
//     padding), the Sylvester stages run as above on every block of b, the
//     row goes through the wave's LDS buffer with true signs, each lane reads
//     its b / 64 coordinates of every block, forms the m-term sums of the
//     Paley factor in increasing block order (the signs are compile-time
//     constants), multiplies by RN32(1 / sqrt(n')) and writes them back, and
//     the quantiser reads the row in its usual layout;
//   * Lloyd-Max codes (OrbitQuant PR #25, "Default changes"; the codebook of
//     the post-rotation marginal): the scale is the row's RMS from the exact
//     sum of squares rounded to float64 (a float64 wavefront sum, recomputed
//     exactly in integers where its error could reach the float32
//     rounding of the RMS), and each code is the number
//     of thresholds below u = v / rho, found by a binary search of |u| over
//     the positive thresholds held in LDS (u <= 0 searches with the next
//     float above |u|, so that a tie goes to the lower level).
#include "oq_internal.h"

#include <type_traits>

#pragma clang fp contract(off)

namespace oq {
namespace {

constexpr int WAVES_PER_WG = 4;

typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned v6u __attribute__((ext_vector_type(6)));

// Partner of this lane in step lg of a butterfly network over the wavefront,
// all on the VALU: lane ^ 1 and lane ^ 2 (quad_perm), then l <-> 7 - l
// within 8 lanes (row_half_mirror), l <-> 15 - l within 16 (row_mirror),
// rows 16 lanes apart (v_permlane16_swap) and halves 32 apart
// (v_permlane32_swap).  After steps 0..k every group of 2^(k+1) lanes has
// met, so a symmetric combination (max, a top-k merge, a commutative add)
// over all six steps leaves the same value on every lane.
__device__ __forceinline__ float xlane(float v, int lg) {
  const int iv = __float_as_int(v);
  switch (lg) {
    case 0: return __int_as_float(__builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, true));   // lane ^ 1
    case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, true));   // lane ^ 2
    case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(iv, 0x141, 0xF, 0xF, true));  // row_half_mirror
    case 3: return __int_as_float(__builtin_amdgcn_mov_dpp(iv, 0x140, 0xF, 0xF, true));  // row_mirror
    case 4: {
      // (value of the even row, value of the odd row) of each row pair
      const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)iv, (uint32_t)iv, false, false);
      return __uint_as_float((__lane_id() & 16) ? r[0] : r[1]);
    }
    default: {
      const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)iv, (uint32_t)iv, false, false);
      return __uint_as_float((__lane_id() & 32) ? r[0] : r[1]);
    }
  }
}

// Wavefront sum of a float64 over the network above, the pair's two values
// added in the same order in both lanes (lower row or half first), so every
// lane ends with the same bits.
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int lg = 0; lg < 4; ++lg) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const float lo = xlane(__uint_as_float((uint32_t)u), lg), hi = xlane(__uint_as_float((uint32_t)(u >> 32)), lg);
    v += __builtin_bit_cast(double, ((uint64_t)__float_as_uint(hi) << 32) | __float_as_uint(lo));
  }
  {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const auto rl = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto rh = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    v = __builtin_bit_cast(double, ((uint64_t)rh[0] << 32) | rl[0]) +
        __builtin_bit_cast(double, ((uint64_t)rh[1] << 32) | rl[1]);
  }
  {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const auto rl = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto rh = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    v = __builtin_bit_cast(double, ((uint64_t)rh[0] << 32) | rl[0]) +
        __builtin_bit_cast(double, ((uint64_t)rh[1] << 32) | rl[1]);
  }
  return v;
}

// True when r (>= 0, float64) lies within 2^-44 r of a float32 rounding
// midpoint, i.e. where a float64 value carrying a few dozen ulps of error
// might round to another float32 than the exact one.
__device__ __forceinline__ bool near_f32_midpoint(double r) {
  const float f = (float)r;
  if (r == 0.0 || !(f < __builtin_inff())) return false;
  const double fu = (double)nextafterf(f, __builtin_inff());
  const double fd = (double)nextafterf(f, 0.0f);
  const double mu = 0.5 * ((double)f + fu), md = 0.5 * ((double)f + fd);  // exact
  return fabs(r - mu) <= r * 0x1p-44 || fabs(r - md) <= r * 0x1p-44;
}

// RN64 of the exact sum of v^2 over a wavefront's n values per lane (the
// entries with act false are skipped).  v = m 2^q with m < 2^24 an integer,
// so v^2 = m^2 2^(2q) is placed at bit 2q + 298 >= 0 of a 608-bit integer
// held as 19 32-bit limbs; the wavefront adds its 32-bit pieces into 64-bit
// LDS counters (at most 4096 pieces of < 2^32 each per counter), every lane
// propagates the carries and rounds the integer to 53 bits, ties to even.
// cnt: 19 uint64 of LDS owned by this wavefront.
template <int SLOTS>
__device__ double exact_sumsq_rn64(const float (&v)[SLOTS][16], const bool (&act)[SLOTS], int lane,
                                   unsigned long long *cnt) {
  if (lane < 19) cnt[lane] = 0ull;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    if (!act[s]) continue;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t u = __float_as_uint(v[s][j]);
      const uint32_t eb = (u >> 23) & 0xFF, mb = u & 0x7FFFFF;
      const uint64_t m = eb ? (uint64_t)(mb | 0x800000u) : (uint64_t)mb;
      if (m == 0) continue;
      const int p = 2 * ((eb ? (int)eb : 1) - 150) + 298;  // bit of m^2's last bit
      const uint64_t t = m * m;                              // < 2^48
      const int i = p >> 5, sh = p & 31;
      const uint64_t lo = t << sh;
      const uint64_t hi = sh ? t >> (64 - sh) : 0ull;
      atomicAdd(&cnt[i], lo & 0xFFFFFFFFull);
      atomicAdd(&cnt[i + 1], lo >> 32);
      if (hi) atomicAdd(&cnt[i + 2], hi);
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  uint32_t L[19];
  uint64_t carry = 0;
#pragma unroll
  for (int k = 0; k < 19; ++k) {
    const uint64_t c = cnt[k] + carry;
    L[k] = (uint32_t)c;
    carry = c >> 32;
  }
  int top = -1;
#pragma unroll
  for (int k = 0; k < 19; ++k)
    if (L[k]) top = k;
  if (top < 0) return 0.0;
  uint32_t a = 0, b = 0, c = 0;  // limbs top, top - 1, top - 2 (zero below limb 0)
  bool sticky = false;
#pragma unroll
  for (int k = 0; k < 19; ++k) {
    if (k == top) a = L[k];
    if (k == top - 1) b = L[k];
    if (k == top - 2) c = L[k];
    if (k < top - 2) sticky |= L[k] != 0;
  }
  const int bpos = 31 - __builtin_clz(a);  // leading bit of the top limb
  const int sdrop = bpos + 12;              // bits of the 96-bit window below the 53 kept
  const uint64_t hi64 = ((uint64_t)a << 32) | b;
  uint64_t mant;
  bool half, rest;
  if (sdrop >= 32) {
    const int s2 = sdrop - 32;
    mant = hi64 >> s2;
    half = s2 > 0 ? ((hi64 >> (s2 - 1)) & 1ull) != 0 : (c >> 31) != 0;
    rest = (s2 > 1 && (hi64 & ((1ull << (s2 - 1)) - 1ull)) != 0) || (s2 > 0 ? c != 0 : (c & 0x7FFFFFFFu) != 0);
  } else {
    mant = (hi64 << (32 - sdrop)) | (c >> sdrop);
    half = ((c >> (sdrop - 1)) & 1u) != 0;
    rest = (c & ((1u << (sdrop - 1)) - 1u)) != 0;
  }
  if (half && (rest || sticky || (mant & 1ull))) ++mant;  // 2^53 is still exact
  return __builtin_ldexp((double)mant, 32 * (top - 2) + sdrop - 298);
}

// Index lane of physical lane `lane` when a Hadamard block spans 2^n lanes.
// Lane-bit stage k flips index bit k and pairs lanes differing by p_k, with
// p = (1, 2, 7, 15) for k < 4 (the DPP patterns) and 2^k above; the physical
// lane is the GF(2) sum of b_k p_k over the index bits b_k, inverted here.
// Bits above the block are unchanged.
__device__ __forceinline__ int index_lane(int lane, int n) {
  const int l0 = lane & 1, l1 = (lane >> 1) & 1, l2 = (lane >> 2) & 1, l3 = (lane >> 3) & 1;
  if (n <= 2) return lane;
  if (n == 3) return (lane & ~7) | (l2 << 2) | ((l1 ^ l2) << 1) | (l0 ^ l2);
  return (lane & ~15) | (l3 << 3) | ((l2 ^ l3) << 2) | ((l1 ^ l2) << 1) | (l0 ^ l2);
}

// v[j] += c * v[j] of the partner lane, 16 values, partner by DPP pattern.
// The s_nop covers the wait states a DPP read needs after a VALU write of
// its source (and after a VALU write of EXEC).
#define OQ_FMAC_DPP(i, CTRL) "v_fmac_f32_dpp %" #i ", %" #i ", %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"
#define OQ_FMAC_DPP16(CTRL)                                                                                   \
  "s_nop 4\n\t" OQ_FMAC_DPP(0, CTRL) OQ_FMAC_DPP(1, CTRL) OQ_FMAC_DPP(2, CTRL) OQ_FMAC_DPP(3, CTRL)           \
      OQ_FMAC_DPP(4, CTRL) OQ_FMAC_DPP(5, CTRL) OQ_FMAC_DPP(6, CTRL) OQ_FMAC_DPP(7, CTRL) OQ_FMAC_DPP(8, CTRL) \
          OQ_FMAC_DPP(9, CTRL) OQ_FMAC_DPP(10, CTRL) OQ_FMAC_DPP(11, CTRL) OQ_FMAC_DPP(12, CTRL)             \
              OQ_FMAC_DPP(13, CTRL) OQ_FMAC_DPP(14, CTRL) OQ_FMAC_DPP(15, CTRL)
#define OQ_V16_OPERANDS(v)                                                                                   \
  "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]), "+v"(v[8]), \
      "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])

template <int K>
__device__ __forceinline__ void dpp_stage(float (&v)[16], float c) {
  if constexpr (K == 0) asm(OQ_FMAC_DPP16("quad_perm:[1,0,3,2]") : OQ_V16_OPERANDS(v) : "v"(c));
  if constexpr (K == 1) asm(OQ_FMAC_DPP16("quad_perm:[2,3,0,1]") : OQ_V16_OPERANDS(v) : "v"(c));
  if constexpr (K == 2) asm(OQ_FMAC_DPP16("row_half_mirror") : OQ_V16_OPERANDS(v) : "v"(c));
  if constexpr (K == 3) asm(OQ_FMAC_DPP16("row_mirror") : OQ_V16_OPERANDS(v) : "v"(c));
}

// Butterflies between lanes 16 (D = 16) or 32 (D = 32) apart, the lower
// lane taking a + b and the upper a - b.  For each pair of values (v[j],
// v[j+1]) one swap leaves, in every lane, the lower and the upper operand of
// one butterfly (value j in the lower lanes of each pair, j + 1 in the upper
// ones); the lane forms the sum and the difference, and the same swap of
// (sum, difference) returns each result to its lane and value.
template <int D>
__device__ __forceinline__ void swap_stage(float (&v)[16]) {
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    const uint32_t a = __float_as_uint(v[j]), b = __float_as_uint(v[j + 1]);
    uint32_t lo, hi;
    if constexpr (D == 16) {
      const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
      lo = r[0];
      hi = r[1];
    } else {
      const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
      lo = r[0];
      hi = r[1];
    }
    const float sum = __uint_as_float(lo) + __uint_as_float(hi);
    const float dif = __uint_as_float(lo) - __uint_as_float(hi);
    if constexpr (D == 16) {
      const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(sum), __float_as_uint(dif), false, false);
      v[j] = __uint_as_float(q[0]);
      v[j + 1] = __uint_as_float(q[1]);
    } else {
      const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(dif), false, false);
      v[j] = __uint_as_float(q[0]);
      v[j + 1] = __uint_as_float(q[1]);
    }
  }
}

// Un-normalised FWHT of each 2^(n+4)-coordinate block; stage order strides
// 1, 2, ..., as in the oracle.  c[k] = -1 where index-lane bit k is set.
// On return lane values carry the sign (-1)^popcount(index lane mod
// 2^min(n, 4)): the DPP stages leave it, the swap stages keep it.
template <int SLOTS>
__device__ __forceinline__ void fwht_row(float (&v)[SLOTS][16], int n, const float (&c)[4]) {
#pragma unroll
  for (int s = 0; s < SLOTS; ++s)
#pragma unroll
    for (int st = 1; st < 16; st <<= 1)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if ((j & st) == 0) {
          const float a = v[s][j], b = v[s][j + st];
          v[s][j] = a + b;
          v[s][j + st] = a - b;
        }
  if (n > 0)
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) dpp_stage<0>(v[s], c[0]);
  if (n > 1)
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) dpp_stage<1>(v[s], c[1]);
  if (n > 2)
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) dpp_stage<2>(v[s], c[2]);
  if (n > 3)
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) dpp_stage<3>(v[s], c[3]);
  if (n > 4)
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) swap_stage<16>(v[s]);
  if (n > 5)
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) swap_stage<32>(v[s]);
}

// Stores the 16 codes of two slots (a: coordinates base..base+15, b: the same
// 1024 further on) of row 32 t + rr in the tiled layout (see k_gemm_fp6.hip):
// the 32 codes of (row, k-half h) form a 192-bit string whose bytes 0..15 sit
// at tile + 16 l and bytes 16..23 at tile + 1024 + 8 l, l = 32 h + rr; this
// lane's 16 codes are its first (base % 32 == 0) or second 96 bits.
// The codes arrive as integer-valued floats (+0 for zero) and are converted
// with v_cvt_scalef32_2xpk16_fp6_f32 (exact: |t| <= 7 or a plane of it),
// which interleaves its sources: field 2k from src0[k], 2k+1 from src1[k].
// part: 0 the codes, 1 the high plane floor(t/8), 2 the low plane
// t - 8 floor(t/8).
__device__ __forceinline__ void store_fp6_pair(const float (&ta)[16], const float (&tb)[16], int part,
                                               uint8_t *tile_base, int rr, int base, bool wa, bool wb) {
  v16f s0, s1;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    float e0 = k < 8 ? ta[2 * k] : tb[2 * k - 16];
    float e1 = k < 8 ? ta[2 * k + 1] : tb[2 * k - 15];
    if (part) {
      const float h0 = __builtin_floorf(e0 * 0.125f), h1 = __builtin_floorf(e1 * 0.125f);
      e0 = part == 1 ? h0 + 0.0f : __builtin_fmaf(h0, -8.0f, e0);
      e1 = part == 1 ? h1 + 0.0f : __builtin_fmaf(h1, -8.0f, e1);
    }
    s0[k] = e0;
    s1[k] = e1;
  }
  const v6u pk = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(s0, s1, 1.0f);
  const int kg = base >> 6, hf = (base >> 5) & 1, j0 = base & 31;
  const int l = 32 * hf + rr;
  uint8_t *tm = tile_base + kg * 1536 + 16 * l;         // bytes 0..15 of the string
  uint8_t *tt = tile_base + kg * 1536 + 1024 + 8 * l;   // bytes 16..23
  // slot b lies 1024 coordinates on: 16 k-groups further
  constexpr int SB = 16 * 1536;
  if (j0 == 0) {
    if (wa) {
      *reinterpret_cast<uint2 *>(tm) = make_uint2(pk[0], pk[1]);
      *reinterpret_cast<uint32_t *>(tm + 8) = pk[2];
    }
    if (wb) {
      *reinterpret_cast<uint2 *>(tm + SB) = make_uint2(pk[3], pk[4]);
      *reinterpret_cast<uint32_t *>(tm + SB + 8) = pk[5];
    }
  } else {
    if (wa) {
      *reinterpret_cast<uint32_t *>(tm + 12) = pk[0];
      *reinterpret_cast<uint2 *>(tt) = make_uint2(pk[1], pk[2]);
    }
    if (wb) {
      *reinterpret_cast<uint32_t *>(tm + SB + 12) = pk[3];
      *reinterpret_cast<uint2 *>(tt + SB) = make_uint2(pk[4], pk[5]);
    }
  }
}

// Factorised rotation shapes on the wave path: m = 12 with b = 64, 128, 256
// (n' = 768, 1536, 3072) and m = 36, 44 with b = 64 (n' = 2304, 2816); a
// lane holds BPL = b / 64 coordinates of every block in the Paley stage.
template <int KM, int SLOTS>
struct KronShape {
  static constexpr int BPL = KM == 12 ? (SLOTS == 3 ? 4 : SLOTS) : 1;
  static constexpr int B = 64 * BPL;
  static_assert(KM * B <= 1024 * SLOTS && KM * B > 1024 * (SLOTS - 1), "width fills the slots");
};

template <int KM>
struct PaleyMasks {
  uint64_t m[KM];
  constexpr PaleyMasks() : m{} {
    for (int r = 0; r < KM; ++r) m[r] = paley_row_mask(KM, r);
  }
};

// Paley stage of the factorised rotation on a row held as index-lane chunks
// (values times sg are the Sylvester outputs): out[c' B + i] = c_h *
// sum_c H_m[c'][c] u[c B + i], the sum in increasing c, through the wave's
// LDS buffer bf (n' floats); on return v holds the rotated row, true signs.
template <int SLOTS, int KM>
__device__ __forceinline__ void kron_paley(float (&v)[SLOTS][16], float *bf, int lane, int il, const bool (&act)[SLOTS],
                                           float sg, float c_h) {
  using KS = KronShape<KM, SLOTS>;
  constexpr int BPL = KS::BPL, B = KS::B;
  constexpr PaleyMasks<KM> H{};
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    if (!act[s]) continue;
    float4 *dst = reinterpret_cast<float4 *>(bf + 1024 * s + 16 * il);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      dst[k] = make_float4(v[s][4 * k] * sg, v[s][4 * k + 1] * sg, v[s][4 * k + 2] * sg, v[s][4 * k + 3] * sg);
  }
  // the wave's own LDS writes are ordered before its reads
  float u[KM][BPL];
#pragma unroll
  for (int c = 0; c < KM; ++c) {
    const float *src = bf + c * B + BPL * lane;
    if constexpr (BPL == 4) {
      const float4 t = *reinterpret_cast<const float4 *>(src);
      u[c][0] = t.x; u[c][1] = t.y; u[c][2] = t.z; u[c][3] = t.w;
    } else if constexpr (BPL == 2) {
      const float2 t = *reinterpret_cast<const float2 *>(src);
      u[c][0] = t.x; u[c][1] = t.y;
    } else {
      u[c][0] = src[0];
    }
  }
#pragma unroll
  for (int cp = 0; cp < KM; ++cp) {
    float y[BPL];
#pragma unroll
    for (int k = 0; k < BPL; ++k) {
      float acc = (H.m[cp] & 1) ? -u[0][k] : u[0][k];
#pragma unroll
      for (int c = 1; c < KM; ++c) acc = ((H.m[cp] >> c) & 1) ? acc - u[c][k] : acc + u[c][k];
      y[k] = acc * c_h;
    }
    float *dst = bf + cp * B + BPL * lane;  // the coordinates this lane read
    if constexpr (BPL == 4) *reinterpret_cast<float4 *>(dst) = make_float4(y[0], y[1], y[2], y[3]);
    else if constexpr (BPL == 2) *reinterpret_cast<float2 *>(dst) = make_float2(y[0], y[1]);
    else dst[0] = y[0];
  }
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const float4 *src = reinterpret_cast<const float4 *>(bf + 1024 * s + 16 * il);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 t = act[s] ? src[k] : make_float4(0.f, 0.f, 0.f, 0.f);
      v[s][4 * k] = t.x; v[s][4 * k + 1] = t.y; v[s][4 * k + 2] = t.z; v[s][4 * k + 3] = t.w;
    }
  }
}

// A group sum p of integer codes (|p| < 2048) as the word the corrected GEMM
// reads: bfloat16 p1 = 8 floor(p / 8) in bits 0-15 and p2 = p - p1 in bits
// 16-31, both exact.
__device__ __forceinline__ uint32_t gsum_pieces(float p) {
  const float p1 = __builtin_floorf(p * 0.125f) * 8.0f;
  return (__float_as_uint(p1) >> 16) | (__float_as_uint(p - p1) & 0xFFFF0000u);
}

// LDS: [offset table: ROUNDS x SLOTS x 4 x 64 lanes x 4 ints]
// [single-copy mode: bf16 sign mask of every input coordinate, SLOTS x 1024 x 2 bytes]
// [per wave: row copies]
// [Lloyd-Max modes: 128 float positive thresholds, 256 float16 levels, when
// they fit in the 160 KiB; otherwise the kernel reads them from global memory]
// Single-copy mode (ONE: one round, absmax or percentile codes): each wave
// keeps one bf16 copy of its row with the signs applied as it is written, so
// the row buffer is half of the two-copy one, and workgroups of 8 waves run
// 4 waves per SIMD (two per CU at d <= 3072); centred (CEN1), 4-wave
// workgroups at 3 per SIMD.
template <int SLOTS, int ROUNDS, bool LM, bool ONE = false, bool CEN1 = false>
struct WaveLds {
  // waves per workgroup: the centred and the Lloyd-Max single-copy bodies
  // need up to 168 registers (3 waves per SIMD), so they run 4-wave
  // workgroups, three per CU
  static constexpr int W = ONE ? (CEN1 || LM ? 4 : 8) : WAVES_PER_WG;
  static constexpr int TABLE = (ROUNDS > 0 ? ROUNDS : 1) * SLOTS * 1024 * 4;
  static constexpr int SMASK = ONE ? SLOTS * 1024 * 2 : 0;
  // one bf16 copy; else 2 copies, float32 if 2 rounds
  static constexpr int ROWBUF = ONE ? 2 * SLOTS * 1024 : (ROUNDS == 2 ? 8 : 4) * SLOTS * 1024;
  static constexpr int LM_OFF = TABLE + SMASK + W * ROWBUF;
  static constexpr bool LM_LDS = LM && LM_OFF + 1024 <= 160 * 1024;
  static constexpr int TOTAL = LM_OFF + (LM_LDS ? 128 * 4 + 256 * 2 : 0);
};

template <int mode>
constexpr bool is_lm_mode() { return mode == OUT_LM4 || mode == OUT_LM8 || mode == OUT_LMF16; }

// mode (OUT_*) is a template argument: one kernel body per output keeps the
// register count of each near what its own path needs.
// KM > 0: the factorised rotation with Paley order KM (ROUNDS 0, h = b, din
// the native width); otherwise din is unused.
template <int SLOTS, int ROUNDS, int mode, bool PCTL, int KM = 0, bool ONE = false, bool CEN1 = false>
__global__ void __launch_bounds__(64 * (ONE ? (CEN1 || is_lm_mode<mode>() ? 4 : 8) : WAVES_PER_WG))
__attribute__((amdgpu_waves_per_eu(ONE ? (CEN1 || is_lm_mode<mode>() ? 3 : 4) : 1)))
rpbh_wave_kernel(const uint16_t *__restrict__ x, int64_t M, int d, int64_t ldx, const int32_t *__restrict__ perm,
                 const int8_t *__restrict__ signs, int h, float c_h, int pow4, int center_arg,
                 float *__restrict__ mean_out, int qmax, void *__restrict__ out, int64_t ld_out_bytes,
                 float *__restrict__ scale_out, PctlArgs pa, LmArgs la, uint32_t *__restrict__ gsum_out, int din) {
  static_assert(KM == 0 || (ROUNDS == 0 && !PCTL && !is_lm_mode<mode>()), "factorised rotation: plain absmax modes");
  static_assert(!ONE || (ROUNDS == 1 && KM == 0), "single copy: one round");
  static_assert(!CEN1 || ONE, "centring is a compile-time choice of the single-copy kernel");
  constexpr bool LM = is_lm_mode<mode>();
  using L = WaveLds<SLOTS, ROUNDS, LM, ONE, CEN1>;
  constexpr int W = L::W;
  const int center = ONE ? (CEN1 ? 1 : 0) : center_arg;  // compile-time in the single-copy kernel
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int *table = reinterpret_cast<int *>(lds_raw);
  uint16_t *smask = reinterpret_cast<uint16_t *>(lds_raw + L::TABLE);
  uint8_t *buf = lds_raw + L::TABLE + L::SMASK + wave * L::ROWBUF;
  const int nlog = __builtin_ctz((unsigned)h) - 4;  // a Hadamard block spans 2^nlog lanes
  const int il = index_lane(lane, nlog);             // this lane holds coordinates 16 il + j of each slot

  // act: this lane's coordinates of slot s exist (index lane); ld: the
  // 16-coordinate chunk it loads exists (its physical chunk, or for the
  // factorised rotation its index-lane chunk of the native row)
  const int ll = KM ? il : lane;
  const int dload = KM ? din : d;
  bool act[SLOTS], ld[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    act[s] = 1024 * s + 16 * il < d;
    ld[s] = 1024 * s + 16 * ll < dload;
  }
  const float c_all = (ROUNDS == 0 || !pow4) ? 1.0f : (ROUNDS == 2 ? c_h * c_h : c_h);  // deferred, exact
  float cst[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) cst[k] = ((il >> k) & 1) ? -1.0f : 1.0f;
  // sign the lane-bit stages leave on this lane's values
  const float sg = (__builtin_popcount(il & ((1 << (nlog < 4 ? nlog : 4)) - 1)) & 1) ? -1.0f : 1.0f;
  const float sgq = KM > 1 ? 1.0f : sg;  // the sign the quantiser sees (the Paley stage removes it)
  const int neg_from = 2 * d;  // first-round byte offsets at or above this hit the -x copy

  // ---- offset table: byte offsets into this wave's [+row | -row] buffer;
  // first-round copies are bf16 (2 bytes), second-round copies float32.
  // Entry (r, s, lane l, j) is coordinate 1024 s + 16 index_lane(l) + j;
  // each task fills 4 consecutive j.
  constexpr int TASKS = (ROUNDS > 0 ? ROUNDS : 0) * SLOTS * 256;
  constexpr int NT = (TASKS + 64 * W - 1) / (64 * W);
  int pv[NT > 0 ? NT : 1][4], sv[NT > 0 ? NT : 1][4];
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    const int q = threadIdx.x + k * 64 * W;
    const int r = q / (SLOTS * 256), rem = q % (SLOTS * 256);
    const int s = rem / 256, l = (rem / 4) % 64, j0 = 4 * (rem % 4);
    const int i0 = 1024 * s + 16 * index_lane(l, nlog) + j0;
    // unconditional loads (index 0 for entries that do not exist, which the
    // table step below zeroes) so that none waits for another
    const int64_t b = (q < TASKS && i0 < d) ? (int64_t)r * d + i0 : 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pv[k][e] = perm[b + e];
      sv[k][e] = signs[b + e];
    }
  }

  const int64_t step = (int64_t)gridDim.x * W;
  // the next row's words are loaded while the current row is processed; the
  // last row of a wave reloads its own words (cached) rather than another
  // row, so the final prefetches of all waves do not meet on one row; lanes
  // beyond the row end read their own first word instead
  uint4 nxt[SLOTS][2];
  auto load_row = [&](int64_t rr) {
    const uint16_t *xr = x + rr * ldx;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const uint4 *src = reinterpret_cast<const uint4 *>(xr + (ld[s] ? 1024 * s + 16 * ll : 0));
      nxt[s][0] = src[0];
      nxt[s][1] = src[1];
    }
  };
  int64_t row = (int64_t)blockIdx.x * W + wave;

  if constexpr (ONE) {
    // the sign mask starts at zero and the scatter index is clamped, so a
    // perm that is not a permutation (outside the caller's contract) gives
    // unspecified codes but no access outside the mask
    for (int i = threadIdx.x; i < SLOTS * 128; i += 64 * W) reinterpret_cast<uint4 *>(smask)[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    const int q = threadIdx.x + k * 64 * W;
    if (q >= TASKS) continue;
    const int r = q / (SLOTS * 256), rem = q % (SLOTS * 256);
    const int s = rem / 256, l = (rem / 4) % 64, jq = rem % 4;
    const int i0 = 1024 * s + 16 * index_lane(l, nlog) + 4 * jq;
    int o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (ONE) {
        // the row copy is signed as it is written: the sign of output i0 + e
        // goes to the input coordinate it gathers (a permutation: every
        // coordinate below d is written once)
        const int pc = min(max(pv[k][e], 0), d - 1);
        o[e] = i0 < d ? 2 * pc : 0;
        if (i0 < d) smask[pc] = sv[k][e] < 0 ? 0x8000u : 0u;
      } else {
        o[e] = i0 < d ? (pv[k][e] + (sv[k][e] < 0 ? d : 0)) * (r == 0 ? 2 : 4) : 0;
      }
    }
    reinterpret_cast<int4 *>(table)[((r * SLOTS + s) * 4 + jq) * 64 + l] = make_int4(o[0], o[1], o[2], o[3]);
  }
  // Lloyd-Max tables: pos[j] = thr[hh - 1 + j], j = 1 .. hh - 1 (the
  // thresholds above the middle one, which is 0), and the levels
  float *lm_pos = reinterpret_cast<float *>(lds_raw + L::LM_OFF);
  uint16_t *lm_lv = reinterpret_cast<uint16_t *>(lds_raw + L::LM_OFF + 512);
  const int hh = LM ? 1 << (la.bits - 1) : 1;
  // the first row is requested once the table's own loads have returned:
  // issued earlier, they would queue behind every wave's row (the chip-wide
  // first burst) and the table would wait for it
  load_row(row < M ? row : M - 1);
  if constexpr (L::LM_LDS) {
    const int t = threadIdx.x;
    if (t >= 1 && t < hh) lm_pos[t] = la.thr[hh - 1 + t];
    if (t < 2 * hh) lm_lv[t] = la.levels[t];
  }
  __syncthreads();

  for (; row < M; row += step) {
    float v[SLOTS][16];
    uint4 raw[SLOTS][2];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      raw[s][0] = nxt[s][0];
      raw[s][1] = nxt[s][1];
    }
    load_row(row + step < M ? row + step : row);

    float m = 0.f;
    if (center) {
      double sum = 0.0;
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const uint32_t w[8] = {raw[s][0].x, raw[s][0].y, raw[s][0].z, raw[s][0].w,
                               raw[s][1].x, raw[s][1].y, raw[s][1].z, raw[s][1].w};
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (ld[s]) sum += (double)bf16_lo(w[k]) + (double)bf16_hi(w[k]);
      }
      sum = wave_sum_d(sum);
      m = (float)(sum / (double)dload);
      if (lane == 0) mean_out[row] = m;
    }

    if (ROUNDS == 0) {  // no lane stages: il == lane
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const uint32_t w[8] = {raw[s][0].x, raw[s][0].y, raw[s][0].z, raw[s][0].w,
                               raw[s][1].x, raw[s][1].y, raw[s][1].z, raw[s][1].w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          v[s][2 * k] = ld[s] ? bf16_lo(w[k]) - m : 0.f;
          v[s][2 * k + 1] = ld[s] ? bf16_hi(w[k]) - m : 0.f;
        }
      }
    }

    if (ROUNDS >= 1) {
      // first-round writer: bf16 +row and -row at natural coordinates, or
      // (single copy) the row with each coordinate's sign applied
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        if (!ld[s]) continue;
        const int p0 = 1024 * s + 16 * lane;
        uint4 *dp = reinterpret_cast<uint4 *>(buf + 2 * p0);
        if constexpr (ONE) {
          const uint4 *sm = reinterpret_cast<const uint4 *>(smask + p0);
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const uint4 w = raw[s][k], m = sm[k];
            dp[k] = make_uint4(w.x ^ m.x, w.y ^ m.y, w.z ^ m.z, w.w ^ m.w);
          }
        } else {
          uint4 *dn = reinterpret_cast<uint4 *>(buf + 2 * (p0 + d));
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const uint4 w = raw[s][k];
            dp[k] = w;
            dn[k] = make_uint4(w.x ^ 0x80008000u, w.y ^ 0x80008000u, w.z ^ 0x80008000u, w.w ^ 0x80008000u);
          }
        }
      }
      // gather (the wave's own LDS writes are ordered before its reads);
      // centering: s x - s m = s RN32(x - m), one rounding.  Lanes past the
      // row end read word 0: their blocks are never stored and are left out
      // of the range
      // (the centring test is hoisted out of the element loop: without it
      // the gather is a read and a shift per element)
      auto gather = [&](auto cc) {
        constexpr bool CEN = decltype(cc)::value;
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
          const int4 *tb = reinterpret_cast<const int4 *>(table) + (s * 4) * 64 + lane;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int4 o4 = tb[k * 64];
            const int oo[4] = {o4.x, o4.y, o4.z, o4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float g = __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t *>(buf + oo[e])) << 16);
              if constexpr (CEN && ONE) {
                // the copy holds s x; s m is m with the coordinate's sign
                // mask added into its sign bit (the same byte offset in the
                // mask table), so s x - s m = s RN32(x - m) as before
                const uint32_t sb = *reinterpret_cast<const uint16_t *>(reinterpret_cast<const uint8_t *>(smask) + oo[e]);
                v[s][4 * k + e] = g - __uint_as_float((sb << 16) + __float_as_uint(m));
              } else if constexpr (CEN) {
                const float mm = oo[e] >= neg_from ? -m : m;
                v[s][4 * k + e] = g - mm;
              } else {
                v[s][4 * k + e] = g;
              }
            }
          }
        }
      };
      if (center) gather(std::true_type{});
      else gather(std::false_type{});
      fwht_row<SLOTS>(v, nlog, cst);
      if (!pow4) {
#pragma unroll
        for (int s = 0; s < SLOTS; ++s)
#pragma unroll
          for (int j = 0; j < 16; ++j) v[s][j] = v[s][j] * c_h;
      }
    }

    if constexpr (KM > 1) {
      fwht_row<SLOTS>(v, nlog, cst);
      kron_paley<SLOTS, KM>(v, reinterpret_cast<float *>(buf), lane, il, act, sg, c_h);
    } else if constexpr (KM == 1) {
      // H_1 = 1: the Sylvester transform of the whole padded row; blocks of
      // 2048 and 4096 add in-register stages across slots (strides 1024,
      // 2048; a lane's slots share its sign), then one multiply by c_h
      fwht_row<SLOTS>(v, nlog, cst);
#pragma unroll
      for (int st = 1; st < SLOTS; st <<= 1)
        if (1024 * 2 * st <= h) {
#pragma unroll
          for (int s = 0; s < SLOTS; ++s)
            if ((s & st) == 0 && s + st < SLOTS) {
#pragma unroll
              for (int j = 0; j < 16; ++j) {
                const float a0 = v[s][j], b0 = v[s + st][j];
                v[s][j] = a0 + b0;
                v[s + st][j] = a0 - b0;
              }
            }
        }
#pragma unroll
      for (int s = 0; s < SLOTS; ++s)
#pragma unroll
        for (int j = 0; j < 16; ++j) v[s][j] = v[s][j] * c_h;
    }

    if (ROUNDS == 2) {
      // second-round writer: float32 +row and -row; the lane's values are
      // sg times the first round's outputs, so sg picks the copy they go to
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        if (!act[s]) continue;
        const int p0 = 1024 * s + 16 * il;
        float4 *dp = reinterpret_cast<float4 *>(buf + 4 * (sg > 0.f ? p0 : p0 + d));
        float4 *dn = reinterpret_cast<float4 *>(buf + 4 * (sg > 0.f ? p0 + d : p0));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          dp[k] = make_float4(v[s][4 * k], v[s][4 * k + 1], v[s][4 * k + 2], v[s][4 * k + 3]);
          dn[k] = make_float4(-v[s][4 * k], -v[s][4 * k + 1], -v[s][4 * k + 2], -v[s][4 * k + 3]);
        }
      }
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const int4 *tb = reinterpret_cast<const int4 *>(table) + ((SLOTS + s) * 4) * 64 + lane;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int4 o4 = tb[k * 64];
          const int oo[4] = {o4.x, o4.y, o4.z, o4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) v[s][4 * k + e] = *reinterpret_cast<const float *>(buf + oo[e]);
        }
      }
      fwht_row<SLOTS>(v, nlog, cst);
      if (!pow4) {
#pragma unroll
        for (int s = 0; s < SLOTS; ++s)
#pragma unroll
          for (int j = 0; j < 16; ++j) v[s][j] = v[s][j] * c_h;
      }
    }

    if (mode == OUT_F32) {
      const float co = c_all * sgq;  // exact: both are powers of two up to sign
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        if (!act[s] || !out) continue;
        float4 *dst = reinterpret_cast<float4 *>(static_cast<char *>(out) + row * ld_out_bytes) + (1024 * s + 16 * il) / 4;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          dst[k] = make_float4(v[s][4 * k] * co, v[s][4 * k + 1] * co, v[s][4 * k + 2] * co, v[s][4 * k + 3] * co);
      }
      continue;
    }

    if constexpr (LM) {
      // rho = RN32(sqrt(S / d)), S the float64 sum of squares of the rotated
      // values (c_all^2 exact); u = RN32(v RN32(1 / rho)) with the deferred
      // factor and lane sign folded into the multiplier (exact)
      double ssp[4] = {0.0, 0.0, 0.0, 0.0};  // four partial sums: shorter dependency chains
#pragma unroll
      for (int s = 0; s < SLOTS; ++s)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (act[s]) ssp[j & 3] += (double)v[s][j] * (double)v[s][j];
      double ss = (ssp[0] + ssp[1]) + (ssp[2] + ssp[3]);
      ss = wave_sum_d(ss);  // the same bits on every lane
      const double c2 = (double)c_all * (double)c_all;
      // Every partial sum above is reached by at most 24 additions of
      // nonnegative terms (16 per lane chain, 2, then 6 across the
      // wavefront), so the square root below is within 16 float64 ulps of the
      // reference value
      // sqrt(RN64(S) / d) of the exact sum S.  Only when it lies within 2^-44
      // of a float32 rounding midpoint can RN32 differ; then S is recomputed
      // exactly (the branch is uniform over the wavefront).
      double r64 = __builtin_sqrt((ss * c2) / (double)d);
      if (near_f32_midpoint(r64))
        r64 = __builtin_sqrt((exact_sumsq_rn64<SLOTS>(v, act, lane, reinterpret_cast<unsigned long long *>(buf)) * c2) /
                             (double)d);
      const float rho = fmaxf((float)r64, 1e-10f);
      if (lane == 0) scale_out[row] = rho;
      const float inv = __fdiv_rn(1.0f, rho) * (c_all * sgq);
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        if (!act[s]) continue;
        // binary search one step at a time across the 16 values, so that
        // their table reads are in flight together
        float key[16];
        bool pos[16];
        int c[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float u = v[s][j] * inv;
          const float au = fabsf(u);
          pos[j] = u > 0.f;
          key[j] = pos[j] ? au : __uint_as_float(__float_as_uint(au) + 1u);
          c[j] = 0;
        }
#pragma unroll
        for (int t = 6; t >= 0; --t) {
          const int st = 1 << t;
          if (st < hh) {
            float pv[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) pv[j] = L::LM_LDS ? lm_pos[c[j] + st] : la.thr[hh - 1 + c[j] + st];
#pragma unroll
            for (int j = 0; j < 16; ++j) c[j] += pv[j] < key[j] ? st : 0;
          }
        }
        int q[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) q[j] = pos[j] ? hh + c[j] : hh - 1 - c[j];
        const int base = 1024 * s + 16 * il;
        char *orow = static_cast<char *>(out) + row * ld_out_bytes;
        if constexpr (mode == OUT_LM8) {
          uint32_t wd[4];
#pragma unroll
          for (int k = 0; k < 4; ++k)
            wd[k] = (uint32_t)q[4 * k] | ((uint32_t)q[4 * k + 1] << 8) | ((uint32_t)q[4 * k + 2] << 16) |
                    ((uint32_t)q[4 * k + 3] << 24);
          *reinterpret_cast<uint4 *>(orow + base) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        } else if constexpr (mode == OUT_LM4) {
          uint32_t wd[2] = {0u, 0u};
#pragma unroll
          for (int j = 0; j < 16; ++j) wd[j >> 3] |= (uint32_t)q[j] << (4 * (j & 7));
          *reinterpret_cast<uint2 *>(orow + base / 2) = make_uint2(wd[0], wd[1]);
        } else {
          // tiled float16: chunk (row / 32, k / 16) with k = base .. base + 15;
          // values k % 16 < 8 go to lane row % 32, the rest to lane 32 + row % 32
          uint32_t hv[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint32_t lo = L::LM_LDS ? lm_lv[q[2 * k]] : la.levels[q[2 * k]];
            const uint32_t hi = L::LM_LDS ? lm_lv[q[2 * k + 1]] : la.levels[q[2 * k + 1]];
            hv[k] = lo | (hi << 16);
          }
          char *chunk = static_cast<char *>(out) + ((row >> 5) * (int64_t)(d >> 4) + (base >> 4)) * 1024;
          const int rr = (int)(row & 31);
          *reinterpret_cast<uint4 *>(chunk + 16 * rr) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
          *reinterpret_cast<uint4 *>(chunk + 16 * (32 + rr)) = make_uint4(hv[4], hv[5], hv[6], hv[7]);
        }
      }
      continue;
    }

    float a = 0.f;
    if constexpr (PCTL) {
      // the four largest magnitudes of the row, t[0] >= .. >= t[3]; a lane's
      // own list first (-1 for coordinates past the row end), then the
      // wavefront merges lists (each insertion keeps the multiset's top four)
      float t[4] = {-1.f, -1.f, -1.f, -1.f};
      auto ins = [&](float xv) {
        t[3] = __builtin_amdgcn_fmed3f(t[3], t[2], xv);
        t[2] = __builtin_amdgcn_fmed3f(t[2], t[1], xv);
        t[1] = __builtin_amdgcn_fmed3f(t[1], t[0], xv);
        t[0] = fmaxf(t[0], xv);
      };
#pragma unroll
      for (int s = 0; s < SLOTS; ++s)
#pragma unroll
        for (int j = 0; j < 16; ++j) ins(act[s] ? fabsf(v[s][j]) : -1.f);
#pragma unroll
      for (int lg = 0; lg < 6; ++lg) {
        const float p0 = xlane(t[0], lg), p1 = xlane(t[1], lg), p2 = xlane(t[2], lg), p3 = xlane(t[3], lg);
        ins(p0);
        ins(p1);
        ins(p2);
        ins(p3);
      }
      const float lo = pa.rank == 4 ? t[3] : (pa.rank == 3 ? t[2] : t[1]);
      const float hi = pa.rank == 4 ? t[2] : (pa.rank == 3 ? t[1] : t[0]);
      const double lo64 = (double)(lo * c_all), hi64 = (double)(hi * c_all);  // c_all: exact
      const double q = lo64 + pa.frac * (hi64 - lo64);
      a = fmaxf((float)((q * pa.gamma) / pa.z), 1e-10f);
    } else {
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        float as = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) as = fmaxf(as, fabsf(v[s][j]));
        if (act[s]) a = fmaxf(a, as);
      }
#pragma unroll
      for (int lg = 0; lg < 6; ++lg) a = fmaxf(a, xlane(a, lg));
      a = fmaxf(a * c_all, 1e-10f);  // c_all is a power of two: exact
    }
    const float fq = (float)qmax;
    const float alpha = __fdiv_rn(a, fq);
    const float inv = __fdiv_rn(fq, a) * (c_all * sgq);  // exact rescale: deferred factor and lane sign
    if (lane == 0) scale_out[row] = alpha;

#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      if (!act[s] || mode == OUT_FP6 || mode == OUT_FP6X2) continue;
      int q[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) q[j] = (int)fminf(fmaxf(__builtin_rintf(v[s][j] * inv), -fq), fq);
      const int base = 1024 * s + 16 * il;
      if (mode == OUT_I8) {
        uint32_t wd[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          wd[k] = (uint32_t)(q[4 * k] & 0xFF) | ((uint32_t)(q[4 * k + 1] & 0xFF) << 8) |
                  ((uint32_t)(q[4 * k + 2] & 0xFF) << 16) | ((uint32_t)(q[4 * k + 3] & 0xFF) << 24);
        *reinterpret_cast<uint4 *>(static_cast<char *>(out) + row * ld_out_bytes + base) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      } else if (mode == OUT_I4) {
        uint32_t wd[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 16; ++j) wd[j >> 3] |= (uint32_t)(q[j] & 0xF) << (4 * (j & 7));
        *reinterpret_cast<uint2 *>(static_cast<char *>(out) + row * ld_out_bytes + base / 2) = make_uint2(wd[0], wd[1]);
      }
    }
    if (mode == OUT_FP6 || mode == OUT_FP6X2) {
      // tiled layout (see k_gemm_fp6.hip): this lane's 16 codes of slot s are
      // the 96-bit string at bit 6*(base % 32) of its half of the k-group.
      // Codes are formed as floats (integer-valued, +0 for zero) and
      // converted two slots at a time with v_cvt_scalef32_2xpk16_fp6_f32,
      // which interleaves its two sources field by field.  With the absmax
      // range no clamp is needed: a = max |v| and inv = RN32(qmax / a) give
      // |v inv| <= qmax (1 + 2^-24)^2, so RNE gives |t| <= qmax; the
      // percentile range clips.
      uint8_t *tb = static_cast<uint8_t *>(out) + ((row >> 5) * (d >> 6)) * 1536;
      const int rr = (int)(row & 31);
      const int64_t pstride = tiled_bytes(M, d);
#pragma unroll
      for (int s0 = 0; s0 < SLOTS; s0 += 2) {
        const bool two = s0 + 1 < SLOTS;
        float ta[16], tbv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          float ra = __builtin_rintf(v[s0][j] * inv);
          float rb = two ? __builtin_rintf(v[two ? s0 + 1 : s0][j] * inv) : 0.0f;
          if constexpr (PCTL) {
            ra = __builtin_amdgcn_fmed3f(ra, -fq, fq);
            rb = __builtin_amdgcn_fmed3f(rb, -fq, fq);
          }
          ta[j] = ra + 0.0f;
          tbv[j] = rb + 0.0f;
        }
        const bool wa = act[s0], wb = two && act[two ? s0 + 1 : s0];
        if (gsum_out) {
          // sums of the codes of each 64-wide group: a lane holds 16 of them;
          // index lanes il ^ 1 and il ^ 2 are physical lanes ^ 1 and ^ 2
          float pa0 = 0.f, pb0 = 0.f;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            pa0 += ta[j];
            pb0 += tbv[j];
          }
          pa0 += xlane(pa0, 0);
          pa0 += xlane(pa0, 1);
          pb0 += xlane(pb0, 0);
          pb0 += xlane(pb0, 1);
          if ((il & 3) == 0) {  // group-major [d / 64][M], as two bfloat16 pieces
            if (wa) gsum_out[(int64_t)((1024 * s0 + 16 * il) >> 6) * M + row] = gsum_pieces(pa0);
            if (wb) gsum_out[(int64_t)((1024 * (s0 + 1) + 16 * il) >> 6) * M + row] = gsum_pieces(pb0);
          }
        }
        if (mode == OUT_FP6) {
          store_fp6_pair(ta, tbv, 0, tb, rr, 1024 * s0 + 16 * il, wa, wb);
        } else {
          store_fp6_pair(ta, tbv, 1, tb, rr, 1024 * s0 + 16 * il, wa, wb);
          store_fp6_pair(ta, tbv, 2, tb + pstride, rr, 1024 * s0 + 16 * il, wa, wb);
        }
      }
    }
  }
}

template <int SLOTS, int ROUNDS, int MODE, bool PCTL, int KM = 0, bool ONE = false, bool CEN1 = false>
hipError_t launch_m(const uint16_t *x, int64_t M, int d, int64_t ldx, const RotArgs &rot, int center, float *mean,
                    int qmax, void *out, int64_t ld_out_bytes, float *scale, const PctlArgs &pa, const LmArgs &la,
                    uint32_t *gsum, hipStream_t stream, int din = 0) {
  using L = WaveLds<SLOTS, ROUNDS, is_lm_mode<MODE>(), ONE, CEN1>;
  const size_t lds = (size_t)L::TOTAL;
  static std::atomic<bool> attr_set[64];
  if (lds > 64 * 1024) {
    const hipError_t e =
        lds_limit_once((const void *)rpbh_wave_kernel<SLOTS, ROUNDS, MODE, PCTL, KM, ONE, CEN1>, (int)lds, attr_set);
    if (e != hipSuccess) return e;
  }
  int64_t grid;
  if constexpr (ONE) {
    // one row per wave while every workgroup fits on the chip at once
    // (workgroups per CU: the LDS allows 160 KiB / TOTAL, the registers
    // two of 8 waves at 4 per SIMD, three of 4 waves at 3 per SIMD), more
    // rows per wave beyond
    const int64_t by_regs = CEN1 || is_lm_mode<MODE>() ? 3 : 2, by_lds = 160 * 1024 / L::TOTAL;
    const int64_t per_cu = by_lds < by_regs ? by_lds : by_regs;
    const int64_t cap = per_cu * device_cus();
    grid = (M + L::W - 1) / L::W;
    if (grid > cap) grid = cap;
  } else {
    // two or more rows per wave so the offset table is amortised
    grid = (M + 2 * L::W - 1) / (2 * L::W);
    if (grid > 1024) grid = 1024;
  }
  if (grid < 1) grid = 1;
  const int h = (ROUNDS || KM) ? rot.block : 16;
  const int pow4 = ROUNDS && ((__builtin_ctz((unsigned)h) & 1) == 0);
  hipLaunchKernelGGL((rpbh_wave_kernel<SLOTS, ROUNDS, MODE, PCTL, KM, ONE, CEN1>), dim3((unsigned)grid), dim3(64 * L::W),
                     lds, stream, x, M, d, ldx, rot.perm, rot.signs, h, rot.c_h, pow4, center, mean, qmax, out,
                     ld_out_bytes, scale, pa, la, gsum, din);
  return hipGetLastError();
}

template <int SLOTS, int ROUNDS, int MODE>
hipError_t launch_p(const uint16_t *x, int64_t M, int d, int64_t ldx, const RotArgs &rot, int center, float *mean,
                    int qmax, void *out, int64_t ld_out_bytes, float *scale, const PctlArgs *pctl, const LmArgs *lm,
                    uint32_t *gsum, hipStream_t stream) {
  const PctlArgs no_p{0, 0.0, 0.0, 1.0};
  if (gsum && MODE != OUT_FP6 && MODE != OUT_FP6X2) return hipErrorInvalidValue;
  const LmArgs no_lm{1, nullptr, nullptr};
  if constexpr (is_lm_mode<MODE>()) {
    if (!lm || pctl) return hipErrorInvalidValue;
    constexpr bool ONE_OK = ROUNDS == 1 && SLOTS <= 3;
    if (ONE_OK && center)
      return launch_m<SLOTS, ROUNDS, MODE, false, 0, ONE_OK, ONE_OK>(x, M, d, ldx, rot, center, mean, qmax, out,
                                                                     ld_out_bytes, scale, no_p, *lm, gsum, stream);
    if (ONE_OK)
      return launch_m<SLOTS, ROUNDS, MODE, false, 0, ONE_OK>(x, M, d, ldx, rot, center, mean, qmax, out, ld_out_bytes,
                                                             scale, no_p, *lm, gsum, stream);
    return launch_m<SLOTS, ROUNDS, MODE, false>(x, M, d, ldx, rot, center, mean, qmax, out, ld_out_bytes, scale, no_p,
                                                *lm, gsum, stream);
  } else {
    if (lm) return hipErrorInvalidValue;
    // one round: the single-copy kernel (centred or not), for the widths
    // and outputs whose registers fit 4 waves per SIMD (128) without spills
    constexpr bool ONE_OK = ROUNDS == 1 && SLOTS <= 3 && !(MODE == OUT_FP6X2 && SLOTS > 1);
    if (pctl) {
      if constexpr (MODE == OUT_F32) return hipErrorInvalidValue;
      else if (ONE_OK && center)
        return launch_m<SLOTS, ROUNDS, MODE, true, 0, ONE_OK, ONE_OK>(x, M, d, ldx, rot, center, mean, qmax, out,
                                                                      ld_out_bytes, scale, *pctl, no_lm, gsum, stream);
      else if (ONE_OK)
        return launch_m<SLOTS, ROUNDS, MODE, true, 0, ONE_OK>(x, M, d, ldx, rot, center, mean, qmax, out,
                                                              ld_out_bytes, scale, *pctl, no_lm, gsum, stream);
      else
        return launch_m<SLOTS, ROUNDS, MODE, true>(x, M, d, ldx, rot, center, mean, qmax, out, ld_out_bytes, scale,
                                                   *pctl, no_lm, gsum, stream);
    }
    if (ONE_OK && center)
      return launch_m<SLOTS, ROUNDS, MODE, false, 0, ONE_OK, ONE_OK>(x, M, d, ldx, rot, center, mean, qmax, out,
                                                                     ld_out_bytes, scale, no_p, no_lm, gsum, stream);
    if (ONE_OK)
      return launch_m<SLOTS, ROUNDS, MODE, false, 0, ONE_OK>(x, M, d, ldx, rot, center, mean, qmax, out, ld_out_bytes,
                                                             scale, no_p, no_lm, gsum, stream);
    return launch_m<SLOTS, ROUNDS, MODE, false>(x, M, d, ldx, rot, center, mean, qmax, out, ld_out_bytes, scale, no_p,
                                                no_lm, gsum, stream);
  }
}

template <int SLOTS, int ROUNDS>
hipError_t launch_w(const uint16_t *x, int64_t M, int d, int64_t ldx, const RotArgs &rot, int center, float *mean,
                    int mode, int qmax, void *out, int64_t ld_out_bytes, float *scale, const PctlArgs *pctl,
                    const LmArgs *lm, uint32_t *gsum, hipStream_t stream) {
#define OQ_MODE_CASE(MD) \
  case MD: return launch_p<SLOTS, ROUNDS, MD>(x, M, d, ldx, rot, center, mean, qmax, out, ld_out_bytes, scale, pctl, lm, gsum, stream);
  switch (mode) {
    OQ_MODE_CASE(OUT_F32)
    OQ_MODE_CASE(OUT_I8)
    OQ_MODE_CASE(OUT_I4)
    OQ_MODE_CASE(OUT_FP6)
    OQ_MODE_CASE(OUT_FP6X2)
    OQ_MODE_CASE(OUT_LM4)
    OQ_MODE_CASE(OUT_LM8)
    OQ_MODE_CASE(OUT_LMF16)
  }
#undef OQ_MODE_CASE
  return hipErrorInvalidValue;
}

template <int SLOTS>
hipError_t launch_r(const uint16_t *x, int64_t M, int d, int64_t ldx, const RotArgs &rot, int center, float *mean,
                    int mode, int qmax, void *out, int64_t ld_out_bytes, float *scale, const PctlArgs *pctl,
                    const LmArgs *lm, uint32_t *gsum, hipStream_t stream) {
  switch (rot.rounds) {
    case 0: return launch_w<SLOTS, 0>(x, M, d, ldx, rot, center, mean, mode, qmax, out, ld_out_bytes, scale, pctl, lm, gsum, stream);
    case 1: return launch_w<SLOTS, 1>(x, M, d, ldx, rot, center, mean, mode, qmax, out, ld_out_bytes, scale, pctl, lm, gsum, stream);
    case 2: return launch_w<SLOTS, 2>(x, M, d, ldx, rot, center, mean, mode, qmax, out, ld_out_bytes, scale, pctl, lm, gsum, stream);
  }
  return hipErrorInvalidValue;
}

template <int SLOTS, int KM>
hipError_t launch_kron_w(const uint16_t *x, int64_t M, int dp, int din, int64_t ldx, const RotArgs &rot, int center,
                         float *mean, int mode, int qmax, void *out, int64_t ld_out_bytes, float *scale,
                         hipStream_t stream) {
  const PctlArgs no_p{0, 0.0, 0.0, 1.0};
  const LmArgs no_lm{1, nullptr, nullptr};
#define OQ_KRON_CASE(MD)                                                                                        \
  case MD:                                                                                                      \
    return launch_m<SLOTS, 0, MD, false, KM>(x, M, dp, ldx, rot, center, mean, qmax, out, ld_out_bytes, scale, \
                                             no_p, no_lm, nullptr, stream, din);
  switch (mode) {
    OQ_KRON_CASE(OUT_F32)
    OQ_KRON_CASE(OUT_I8)
    OQ_KRON_CASE(OUT_I4)
    OQ_KRON_CASE(OUT_FP6)
    OQ_KRON_CASE(OUT_FP6X2)
  }
#undef OQ_KRON_CASE
  return hipErrorInvalidValue;
}

}  // namespace

bool rpbh_wave_kron_supported(int km, int b, int din) {
  if (din % 16 != 0) return false;
  return (km == 1 && b >= 16 && b <= 4096 && (b <= 1024 || b == 2048 || b == 4096)) ||
         (km == 12 && (b == 64 || b == 128 || b == 256)) || ((km == 36 || km == 44) && b == 64);
}

hipError_t launch_rpbh_wave_kron(const uint16_t *x, int64_t M, int din, int64_t ldx, const RotArgs &rot, int center,
                                 float *mean, int mode, int qmax, void *out, int64_t ld_out_bytes, float *scale,
                                 hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int km = rot.kron_m, b = rot.block;
  if (!rpbh_wave_kron_supported(km, b, din)) return hipErrorInvalidValue;
  const int dp = km * b;
  if (km == 1 && b <= 1024)
    return launch_kron_w<1, 1>(x, M, dp, din, ldx, rot, center, mean, mode, qmax, out, ld_out_bytes, scale, stream);
  if (km == 1 && b == 2048)
    return launch_kron_w<2, 1>(x, M, dp, din, ldx, rot, center, mean, mode, qmax, out, ld_out_bytes, scale, stream);
  if (km == 1)
    return launch_kron_w<4, 1>(x, M, dp, din, ldx, rot, center, mean, mode, qmax, out, ld_out_bytes, scale, stream);
  if (km == 12 && b == 64)
    return launch_kron_w<1, 12>(x, M, dp, din, ldx, rot, center, mean, mode, qmax, out, ld_out_bytes, scale, stream);
  if (km == 12 && b == 128)
    return launch_kron_w<2, 12>(x, M, dp, din, ldx, rot, center, mean, mode, qmax, out, ld_out_bytes, scale, stream);
  if (km == 12)
    return launch_kron_w<3, 12>(x, M, dp, din, ldx, rot, center, mean, mode, qmax, out, ld_out_bytes, scale, stream);
  if (km == 36)
    return launch_kron_w<3, 36>(x, M, dp, din, ldx, rot, center, mean, mode, qmax, out, ld_out_bytes, scale, stream);
  return launch_kron_w<3, 44>(x, M, dp, din, ldx, rot, center, mean, mode, qmax, out, ld_out_bytes, scale, stream);
}

bool rpbh_wave_supported(int d) { return d >= 16 && d <= 4096 && d % 16 == 0; }

hipError_t launch_rpbh_wave(const uint16_t *x, int64_t M, int d, int64_t ldx, const RotArgs &rot, int center,
                            float *mean, int mode, int qmax, void *out, int64_t ld_out_bytes, float *scale,
                            hipStream_t stream, const PctlArgs *pctl, const LmArgs *lm, uint32_t *gsum) {
  if (M == 0) return hipSuccess;
  if (pctl && (pctl->rank < 2 || pctl->rank > 4)) return hipErrorInvalidValue;
  if (lm && (lm->bits < 1 || lm->bits > 8 || (mode == OUT_LM4 && lm->bits > 4))) return hipErrorInvalidValue;
  switch ((d + 1023) / 1024) {
    case 1: return launch_r<1>(x, M, d, ldx, rot, center, mean, mode, qmax, out, ld_out_bytes, scale, pctl, lm, gsum, stream);
    case 2: return launch_r<2>(x, M, d, ldx, rot, center, mean, mode, qmax, out, ld_out_bytes, scale, pctl, lm, gsum, stream);
    case 3: return launch_r<3>(x, M, d, ldx, rot, center, mean, mode, qmax, out, ld_out_bytes, scale, pctl, lm, gsum, stream);
    case 4: return launch_r<4>(x, M, d, ldx, rot, center, mean, mode, qmax, out, ld_out_bytes, scale, pctl, lm, gsum, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace oq
