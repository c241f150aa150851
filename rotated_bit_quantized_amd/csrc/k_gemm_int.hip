// K3/K4: integer-coded activations x packed INT4 weights with the fp32
// per-group scale and rank-1 epilogue, gfx950 int8 MFMA.
//
// y[t][o] = bf16( a_scale[t] * sum_g w_scale[o][g] * acc_g[t][o]
//                 + mean[t] * w1[o] + bias[o] )          CentriQ Eq. 5 / Eq. 9
// acc_g = exact int32 sum over the g-th group of input columns
// (CentriQ Sec. 3 Eq. 2: one weight scale per row and group of columns).
//
// Tiling: 256 threads = 4 wavefronts in a 2 x 2 grid; each wavefront owns a
// 64 x 64 output tile = 2 x 2 MFMA 32x32 tiles.  For every 32-deep k step a
// lane feeds v_mfma_i32_32x32x32_i8 with 16 consecutive k of one row
// (lanes 0-31: rows 0-31, k 0-15; lanes 32-63: k 16-31), unpacking 4-bit
// codes to int8 in registers; the operands (and group scales) of the step
// seven ahead are loaded meanwhile into a ring of registers.  After the last
// k step of a group each int32 accumulator is converted and folded into the
// fp32 sum with its column's group scale; the output layout of a 32x32 MFMA
// tile puts column l%32 in lane l, so each lane needs one scale per tile per
// group.  The epilogue takes the workgroup's row scales and means from LDS.
#include "oq_internal.h"

#include <type_traits>

namespace oq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 8 bytes of 4-bit two's-complement codes -> 16 sign-extended int8, same order
__device__ __forceinline__ v4i unpack16(uint2 p) {
  v4i r;
  const uint32_t src[2] = {p.x, p.y};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t lo = src[h] & 0x0F0F0F0Fu;          // codes 0, 2, 4, 6
    uint32_t hi = (src[h] >> 4) & 0x0F0F0F0Fu;   // codes 1, 3, 5, 7
    // per byte z in [0,15] -> z - 16 [z >= 8] without cross-byte borrow
    lo = ((lo ^ 0x88888888u) - 0x08080808u) ^ 0x80808080u;
    hi = ((hi ^ 0x88888888u) - 0x08080808u) ^ 0x80808080u;
    r[2 * h] = (int)__builtin_amdgcn_perm(hi, lo, 0x05010400u);
    r[2 * h + 1] = (int)__builtin_amdgcn_perm(hi, lo, 0x07030602u);
  }
  return r;
}

// SPLIT: workgroup z of gridDim.z takes the groups [z c, min((z + 1) c, K /
// group)) with c = ceil((K / group) / gridDim.z) and writes its float32 sum
// of s_g acc_g to part[z][M][N] (no epilogue); split_reduce_kernel adds the
// partial sums in z order and applies the epilogue.
template <bool A_NIB, bool SPLIT>
__global__ void __launch_bounds__(256)
gemm_int_kernel(const uint8_t *__restrict__ qa, int64_t lda, const float *__restrict__ a_scale,
                int64_t M, int K, const uint8_t *__restrict__ w, const float *__restrict__ w_scale,
                int N, int group, const float *__restrict__ mean, const float *__restrict__ w1,
                const float *__restrict__ bias, uint16_t *__restrict__ y, int64_t ldy, float *__restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t m0 = (int64_t)blockIdx.y * 128 + (wave >> 1) * 64;
  const int n0 = blockIdx.x * 128 + (wave & 1) * 64;
  const int r32 = lane & 31;
  const int half = lane >> 5;
  const int Gall = K / group;
  // this workgroup's groups [gb, ge)
  int gb = 0, ge = Gall;
  if constexpr (SPLIT) {
    const int c = (Gall + (int)gridDim.z - 1) / (int)gridDim.z;
    gb = (int)blockIdx.z * c;
    ge = gb + c < Gall ? gb + c : Gall;
    if (gb > ge) gb = ge;
  }
  const int G = ge;  // loads and folds stop at group ge

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

  // the workgroup's 128 row scales and means, loaded now and used after the
  // main loop (through LDS: a lane's 16 values lie in 16 different rows)
  float pre_a = 0.f, pre_m = 0.f;
  if (threadIdx.x < 128) {
    int64_t row = (int64_t)blockIdx.y * 128 + threadIdx.x;
    if (row > M - 1) row = M - 1;
    pre_a = a_scale[row];
    if (mean) pre_m = mean[row];
  }
  float w1v[2] = {0.f, 0.f}, bv[2] = {0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = n0 + 32 * j + r32;
    if (col < N) {
      if (mean) w1v[j] = w1[col];
      if (bias) bv[j] = bias[col];
    }
  }

  float F[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) F[i][j][r] = 0.f;

  // k runs in steps of 32 (group / 32 steps per group); the operands of step
  // s + D - 1 are loaded while step s computes, from a ring of D register
  // sets, so that the latency of the plain global loads is covered
  constexpr int D = 8;
  const int SPG = group / 32, S = (ge - gb) * SPG, st0 = gb * SPG;
  typedef typename std::conditional<A_NIB, uint2, uint4>::type RawA;
  RawA ra[D][2];
  uint2 rw[D][2];
  float rs[D][2];  // the group scales of each loaded step's group
  int gl = gb, kl = 0;  // group and step within it of the next load (loads run in step order)
  // Loads are unconditional, from rows and steps clamped into range: rows
  // past M or N only feed outputs that are never stored, and steps past the
  // end are never computed, so no branch splits the copy queue.
  int64_t arc[2];
  int64_t wrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    arc[i] = (aok[i] ? arow[i] : M - 1) * lda;
    wrc[i] = (int64_t)(wok[i] ? wrow[i] : N - 1) * (K / 2);
  }
  const float *wsc0 = w_scale + (int64_t)(wok[0] ? wrow[0] : N - 1) * Gall;  // rows of K / group scales
  const float *wsc1 = w_scale + (int64_t)(wok[1] ? wrow[1] : N - 1) * Gall;
  auto load = [&](int slot, int st) {
    const int k = 32 * (st0 + (st < S ? st : S - 1)) + 16 * half;
    const int gq = gl < G ? gl : G - 1;
    rs[slot][0] = wsc0[gq];
    rs[slot][1] = wsc1[gq];
    if (++kl == SPG) {
      kl = 0;
      ++gl;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (A_NIB) ra[slot][i] = *reinterpret_cast<const uint2 *>(qa + arc[i] + k / 2);
      else ra[slot][i] = *reinterpret_cast<const uint4 *>(qa + arc[i] + k);
      rw[slot][i] = *reinterpret_cast<const uint2 *>(w + wrc[i] + k / 2);
    }
  };
  v16i acc[2][2];
  if (S > 0) {
#pragma unroll
  for (int q = 0; q < D - 1; ++q) load(q, q);
  for (int s0 = 0; s0 < S; s0 += D) {
#pragma unroll
    for (int q = 0; q < D; ++q) {
      const int st = s0 + q;
      load((q + D - 1) % D, st + D - 1);
      if (st < S) {
        const int kk = st % SPG;
        if (kk == 0) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = (v16i){};
        }
        v4i A[2], B[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if constexpr (A_NIB) {
            A[i] = unpack16(ra[q][i]);
          } else {
            const uint4 p = ra[q][i];
            A[i] = (v4i){(int)p.x, (int)p.y, (int)p.z, (int)p.w};
          }
          B[i] = unpack16(rw[q][i]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[i], B[j], acc[i][j], 0, 0, 0);
        if (kk == SPG - 1) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) F[i][j][r] = __builtin_fmaf(rs[q][j], (float)acc[i][j][r], F[i][j][r]);
        }
      }
    }
  }
  }

  if constexpr (SPLIT) {
    float *pz = part + (int64_t)blockIdx.z * M * N;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + 32 * i + (r >> 2) * 8 + half * 4 + (r & 3);
        if (row >= M) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + 32 * j + r32;
          if (col < N) pz[row * N + col] = F[i][j][r];
        }
      }
    }
    return;
  }

  __shared__ float s_alpha[128], s_mean[128];
  if (threadIdx.x < 128) {
    s_alpha[threadIdx.x] = pre_a;
    s_mean[threadIdx.x] = pre_m;
  }
  __syncthreads();
  const int rw0 = (wave >> 1) * 64;  // this wave's first row within the workgroup
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = rw0 + 32 * i + (r >> 2) * 8 + half * 4 + (r & 3);
      const int64_t row = m0 + 32 * i + (r >> 2) * 8 + half * 4 + (r & 3);
      if (row >= M) continue;
      const float al = s_alpha[rl];
      const float mu = s_mean[rl];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + 32 * j + r32;
        if (col >= N) continue;
        float v = al * F[i][j][r];
        if (mean) v = __builtin_fmaf(mu, w1v[j], v);
        if (bias) v = v + bv[j];
        y[row * ldy + col] = f32_to_bf16_rne(v);
      }
    }
  }
}

// Small products of 8-bit activations (fewer 128 x 128 output tiles than
// half the CUs, K <= 4096): a workgroup of 4 wavefronts per 32 x 32 output
// tile, each wavefront one 16 x 16 quarter over the whole of K with
// v_mfma_i32_16x16x64_i8, groups in order, the same fold and epilogue
// arithmetic as gemm_int_kernel (the integer group sums are exact whatever
// the MFMA shape), so the two give identical bits.  The tile's operands go
// through LDS in chunks of 1024 k read with coalesced 16-byte loads (each
// row's chunk is one contiguous run; a wavefront loads 8 activation rows and
// 8 weight rows, 16 loads a lane, all in flight at once); the next chunk's
// loads are issued before the current chunk is computed.  LDS rows are
// padded (1040 and 528 bytes) so the fragment reads are free of bank
// conflicts.  256 x 1024 x 1024 then runs 256 workgroups, one round trip to
// memory each.
constexpr int SM_KC = 1024;              // k per chunk
constexpr int SM_AROW = SM_KC + 16;      // LDS bytes per activation row of a chunk
constexpr int SM_WROW = SM_KC / 2 + 16;  // LDS bytes per weight row (4-bit codes)
constexpr int SM_NG = SM_KC / 32;        // most groups that end in one chunk
constexpr int SM_LDS = 32 * SM_AROW + 32 * SM_WROW + (SM_NG * 32 + 2 * 32) * 4;

__global__ void __launch_bounds__(256)
gemm_int_small_kernel(const uint8_t *__restrict__ qa, int64_t lda, const float *__restrict__ a_scale, int64_t M,
                      int K, const uint8_t *__restrict__ w, const float *__restrict__ w_scale, int N, int group,
                      const float *__restrict__ mean, const float *__restrict__ w1, const float *__restrict__ bias,
                      uint16_t *__restrict__ y, int64_t ldy) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t *la = smem;
  uint8_t *lw = smem + 32 * SM_AROW;
  float *ls = reinterpret_cast<float *>(smem + 32 * SM_AROW + 32 * SM_WROW);  // [group - first of chunk][column]
  float *l_alpha = ls + SM_NG * 32, *l_mean = l_alpha + 32;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t m0 = (int64_t)blockIdx.y * 32;
  const int n0 = blockIdx.x * 32;
  const int r16 = lane & 15, q = lane >> 4;        // fragment row (column) and k quarter
  const int wr = 16 * (wave >> 1), wc = 16 * (wave & 1);  // this wave's quarter of the tile
  const int G = K / group, SPG = group / 32;

  // epilogue operands; the row scales and means through LDS (a lane's 4
  // outputs lie in 4 rows)
  if (t < 32) {
    const int64_t row = m0 + t < M ? m0 + t : M - 1;
    l_alpha[t] = a_scale[row];
    l_mean[t] = mean ? mean[row] : 0.f;
  }
  const int col = n0 + wc + r16;
  const float w1v = (mean && col < N) ? w1[col] : 0.f;
  const float bv = (bias && col < N) ? bias[col] : 0.f;

  // chunk loads, unconditional from clamped rows and offsets (bytes past the
  // chunk's end and rows past M or N are loaded but never read): wave v's
  // activation load i covers row 8 v + i, bytes 16 lane of its chunk; its
  // weight load i covers row 8 v + 2 i + lane / 32, bytes 16 (lane % 32);
  // scale load j covers group 8 j + t / 32 of those ending in the chunk,
  // column t % 32.  Native vectors: a struct copy from global memory would
  // stay in scratch.
  u32x4 ra[8], rw[4];
  float rs[4];
#define OQ_SMALL_LOAD(KN)                                                                                    \
  do {                                                                                                       \
    const int kn_ = (KN), L_ = K - kn_ < SM_KC ? K - kn_ : SM_KC;                                            \
    const int ba_ = 16 * lane < L_ ? 16 * lane : L_ - 16;                                                    \
    const int bw_ = 16 * (lane & 31) < L_ / 2 ? 16 * (lane & 31) : L_ / 2 - 16;                              \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                                          \
      int64_t row = m0 + 8 * wave + i;                                                                       \
      if (row > M - 1) row = M - 1;                                                                          \
      ra[i] = *reinterpret_cast<const u32x4 *>(qa + row * lda + kn_ + ba_);                                  \
    }                                                                                                        \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                                          \
      int wrow = n0 + 8 * wave + 2 * i + (lane >> 5);                                                        \
      if (wrow > N - 1) wrow = N - 1;                                                                        \
      rw[i] = *reinterpret_cast<const u32x4 *>(w + (int64_t)wrow * (K / 2) + kn_ / 2 + bw_);                 \
    }                                                                                                        \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                                          \
      int c = n0 + (t & 31), g = kn_ / group + 8 * j + (t >> 5);                                             \
      if (c > N - 1) c = N - 1;                                                                              \
      if (g > G - 1) g = G - 1;                                                                              \
      rs[j] = w_scale[(int64_t)c * G + g];                                                                   \
    }                                                                                                        \
  } while (0)

  float F[4] = {0.f, 0.f, 0.f, 0.f};
  v4i acc = (v4i){};
  OQ_SMALL_LOAD(0);
  for (int kc = 0; kc < K; kc += SM_KC) {
    if (kc > 0) __syncthreads();  // every wave's reads of the previous chunk are done
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4 *>(la + (8 * wave + i) * SM_AROW + 16 * lane) = ra[i];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4 *>(lw + (8 * wave + 2 * i + (lane >> 5)) * SM_WROW + 16 * (lane & 31)) = rw[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) ls[t + 256 * j] = rs[j];
    __syncthreads();
    if (kc + SM_KC < K) OQ_SMALL_LOAD(kc + SM_KC);
    const int steps = (K - kc < SM_KC ? K - kc : SM_KC) / 64;
    const int gq0 = kc / group;
    // fragments of step s + 1 are read while step s multiplies: lane (r, q)
    // holds k 16 q .. 16 q + 15 of the step's 64 for row (column) r
    const uint8_t *fa = la + (wr + r16) * SM_AROW + 16 * q, *fw = lw + (wc + r16) * SM_WROW + 8 * q;
    u32x4 pa = *reinterpret_cast<const u32x4 *>(fa);
    uint2 pw = *reinterpret_cast<const uint2 *>(fw);
    for (int s = 0; s < steps; ++s) {
      const int sn = s + 1 < steps ? s + 1 : s;
      const u32x4 na = *reinterpret_cast<const u32x4 *>(fa + 64 * sn);
      const uint2 nw = *reinterpret_cast<const uint2 *>(fw + 32 * sn);
      const v4i A = __builtin_bit_cast(v4i, pa), B = unpack16(pw);
      pa = na;
      pw = nw;
      if (SPG == 1) {
        // groups of 32: the step's two groups in turn, each MFMA with the
        // other group's activation bytes (lanes of the other k halves) zeroed
        const v4i Z = (v4i){};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8((q >> 1) == hh ? A : Z, B, acc, 0, 0, 0);
          const float sw = ls[(2 * s + hh) * 32 + wc + r16];
#pragma unroll
          for (int e = 0; e < 4; ++e) F[e] = __builtin_fmaf(sw, (float)acc[e], F[e]);
          acc = (v4i){};
        }
      } else {
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, acc, 0, 0, 0);
        const int k_end = kc + 64 * s + 64;
        if (k_end % group == 0) {
          const float sw = ls[(k_end / group - 1 - gq0) * 32 + wc + r16];
#pragma unroll
          for (int e = 0; e < 4; ++e) F[e] = __builtin_fmaf(sw, (float)acc[e], F[e]);
          acc = (v4i){};
        }
      }
    }
  }
#undef OQ_SMALL_LOAD

  // y = a_scale * F + mean * w1 + bias (gemm_int_kernel's order); lane (r,
  // q) holds rows 4 q + e of column r of the wave's quarter
  if (col >= N) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int rl = wr + 4 * q + e;
    const int64_t row = m0 + rl;
    if (row >= M) continue;
    float v = l_alpha[rl] * F[e];
    if (mean) v = __builtin_fmaf(l_mean[rl], w1v, v);
    if (bias) v = v + bv;
    y[row * ldy + col] = f32_to_bf16_rne(v);
  }
}

// y = bf16( a_scale[t] (part[0] + part[1] + ... + part[S-1]) + mean[t] w1[o]
// + bias[o] ), the partial sums added in split order; four outputs a thread.
__global__ void __launch_bounds__(256)
split_reduce_kernel(const float *__restrict__ part, int S, int64_t M, int N, const float *__restrict__ a_scale,
                    const float *__restrict__ mean, const float *__restrict__ w1, const float *__restrict__ bias,
                    uint16_t *__restrict__ y, int64_t ldy) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // quad of outputs
  const int nq = (N + 3) / 4;
  const int64_t row = q / nq;
  if (row >= M) return;
  const int c0 = (int)(q % nq) * 4;
  float F[4] = {0.f, 0.f, 0.f, 0.f};
  const bool quad = (N & 3) == 0;  // then every quad is whole and 16-byte aligned
  for (int z = 0; z < S; ++z) {
    const float *pz = part + ((int64_t)z * M + row) * N + c0;
    float p[4];
    if (quad) {
      const float4 v = *reinterpret_cast<const float4 *>(pz);
      p[0] = v.x, p[1] = v.y, p[2] = v.z, p[3] = v.w;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) p[c] = c0 + c < N ? pz[c] : 0.f;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) F[c] = z == 0 ? p[c] : F[c] + p[c];
  }
  const float al = a_scale[row];
  const float mu = mean ? mean[row] : 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int col = c0 + c;
    if (col >= N) continue;
    float v = al * F[c];
    if (mean) v = __builtin_fmaf(mu, w1[col], v);
    if (bias) v = v + bias[col];
    y[row * ldy + col] = f32_to_bf16_rne(v);
  }
}

}  // namespace

hipError_t launch_gemm_int(const void *qa, int64_t lda_bytes, int a_is_nibble, const float *a_scale,
                           int64_t M, int K, const uint8_t *w, const float *w_scale, int N, int group,
                           const float *mean, const float *w1, const float *bias, uint16_t *y,
                           int64_t ldy, hipStream_t stream, void *ws, size_t ws_bytes) {
  if (M == 0 || N == 0) return hipSuccess;
  if (!a_is_nibble && int_gemm_small(M, N, K)) {
    hipLaunchKernelGGL(gemm_int_small_kernel, dim3((unsigned)((N + 31) / 32), (unsigned)((M + 31) / 32)), dim3(256),
                       SM_LDS, stream, (const uint8_t *)qa, lda_bytes, a_scale, M, K, w, w_scale, N, group, mean, w1,
                       bias, y, ldy);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((N + 127) / 128), (unsigned)((M + 127) / 128));
  const int S = a_is_nibble ? 1 : int_gemm_splits(M, N, K, group);
  if (S > 1 && ws && ws_bytes >= (size_t)S * (size_t)M * (size_t)N * 4) {
    float *part = static_cast<float *>(ws);
    grid.z = (unsigned)S;
    hipLaunchKernelGGL((gemm_int_kernel<false, true>), grid, dim3(256), 0, stream, (const uint8_t *)qa, lda_bytes,
                       a_scale, M, K, w, w_scale, N, group, mean, w1, bias, y, ldy, part);
    const int64_t quads = M * ((N + 3) / 4);
    hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, stream, part, S, M,
                       N, a_scale, mean, w1, bias, y, ldy);
    return hipGetLastError();
  }
  if (a_is_nibble)
    hipLaunchKernelGGL((gemm_int_kernel<true, false>), grid, dim3(256), 0, stream, (const uint8_t *)qa, lda_bytes,
                       a_scale, M, K, w, w_scale, N, group, mean, w1, bias, y, ldy, nullptr);
  else
    hipLaunchKernelGGL((gemm_int_kernel<false, false>), grid, dim3(256), 0, stream, (const uint8_t *)qa, lda_bytes,
                       a_scale, M, K, w, w_scale, N, group, mean, w1, bias, y, ldy, nullptr);
  return hipGetLastError();
}

}  // namespace oq
