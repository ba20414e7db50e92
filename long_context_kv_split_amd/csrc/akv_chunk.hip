// Prefill-chunk attention: Tq causal queries per sequence over the two-tier
// history, on 16x16x32 matrix-core tiles (ActiveKV, "Context beyond VRAM",
// "What I built": exact recent tier + compact older tier, merged with exact
// attention arithmetic; the compact tier is read through the pre-rotated query
// of the QuantForge walkthrough, section 1).
//
// Rows of one kv head are (query, head) pairs r = tau * G + g.  A workgroup
// (4 waves x 32 rows) takes 128 consecutive rows and one split (a run of
// whole blocks of one tier).  Each 64-token block is expanded once into LDS
// and used by all 128 rows:
//   compressed tier: K[token][dim] = C[code] * scale in fp32, stored as fp16
//     hi + lo parts, and the transposed V^T[dim][token] = fp16(C[code] *
//     scale).  The query is rotated by the Walsh-Hadamard butterflies in fp32
//     and split into fp16 hi + lo parts; a score is Khi.Qhi + Khi.Qlo +
//     Klo.Qhi (three tiles), about 22 significant bits, so the log-sum-exp
//     keeps fp32-like accuracy on short or outlier-heavy histories;
//   exact tier: bf16 K rows and transposed bf16 V with the bf16 query (exact
//     products, fp32 sums); the last Tq exact tokens are the chunk itself and
//     query tau sees chunk tokens <= tau.
// Per wave:  S^T[token][row] = K_tile x Q^T  and  O^T[dim][row] += V^T x P^T,
// with an online softmax per row; every wave owns its rows, so a split's
// partial (normalized output, log-sum-exp) is written straight from
// registers.  A second kernel merges each row's splits in ascending order:
// compressed-tier splits in rotated space, one inverse rotation, exact-tier
// splits, then both tiers.
#include "akv_common.h"
#include "akv_params.h"

namespace akv {

constexpr int kCWaves = 4;
constexpr int kCThreads = 64 * kCWaves;
constexpr int kRT = 2;                       // 16-row tiles per wave
constexpr int kRowsPerWG = 16 * kRT * kCWaves;
static_assert(kRowsPerWG == AKV_CHUNK_ROWS, "the split planner counts row groups of AKV_CHUNK_ROWS");

__device__ inline float4v cmfma16(half8 a, half8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ inline float4v cmfma16bf(bf16x8 a, bf16x8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline float cxor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ inline float cxor16(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 16) ? r[0] : r[1]);
}

__device__ inline float half_bits(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

// The value of an fp32 expression, rounded to fp32 and opaque to the
// optimizer.  An fp16 hi + lo split must convert hi, and subtract it, from
// one fp32 value: left to itself the backend folds (_Float16)(a * b) into a
// single-rounding mixed multiply for some uses only, so on fp16 ties hi and
// the hi that lo was taken from differ by one ulp.
__device__ inline float fp32_pinned(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// LDS layout of one staged block.  K rows (64 tokens x D 16-bit values, no
// padding) hold 16-byte chunk c of token t at chunk position c ^ kswz(t): the
// 16 tokens an MFMA operand read touches (t = 8u + v + const) and the 16 chunks
// a staging write touches then fall in distinct banks.  V^T rows (D dims x 64
// tokens) have a 144-byte pitch, so 16 consecutive dims start in distinct
// banks.
template <int D>
struct ChunkLds {
  static constexpr int CPR = D / 8;            // 16-byte chunks per K row
  static constexpr int KP = D * 2;
  static constexpr int VP = 64 * 2 + 16;
  static constexpr int K_BYTES = 64 * KP;
  static constexpr int V_BYTES = D * VP;
  static constexpr int KLO = K_BYTES;           // compressed tier: K lo parts
  static constexpr int V0 = 2 * K_BYTES;
  static constexpr int LEV = V0 + V_BYTES;      // 16 fp32 levels
  static constexpr int BYTES = LEV + 64;
};

template <int D>
__device__ inline int kchunk_off(int t, int c) {
  const int h = ((t & 3) << 2) | ((t >> 3) & 3);
  return t * ChunkLds<D>::KP + 16 * (c ^ (h & (ChunkLds<D>::CPR - 1)));
}

// ---- expand one compressed block (64 tokens, nvalid of them real) into LDS
template <int D>
__device__ inline void stage_quant_block(const AttnParams& p, int pb, int kv, int nvalid, unsigned char* smem) {
  constexpr int M = D / 32, VP = ChunkLds<D>::VP;
  const int tid = threadIdx.x;
  const float* lev = reinterpret_cast<const float*>(smem + ChunkLds<D>::LEV);
  const size_t slab = (size_t)pb * p.Hkv + kv;
  const unsigned char* kcs = p.kc + slab * (32 * D);
  const unsigned char* vcs = p.vc + slab * (32 * D);
  const uint16_t* kss = p.ks + slab * (2 * D);
  const uint16_t* vss = p.vs + slab * (2 * D);
  // K: code dword w of a token row holds dims 32*(w % M) + 8*(w / M) + 0..7
  constexpr int KQ = D / 32;  // 16-byte code loads per token row
  for (int ci = tid; ci < 64 * KQ; ci += kCThreads) {
    const int tok = ci / KQ, ch = ci - tok * KQ;
    const u32x4 x = *reinterpret_cast<const u32x4*>(kcs + tok * (D / 2) + 16 * ch);
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      const int wi = 4 * ch + wd, m = wi % M, a = wi / M;
      const float s = tok < nvalid ? half_bits(kss[m * 64 + tok]) : 0.0f;
      half8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = fp32_pinned(lev[(x[wd] >> (4 * e)) & 15] * s);
        hi[e] = (_Float16)v;
        lo[e] = (_Float16)(v - (float)hi[e]);
      }
      const int off = kchunk_off<D>(tok, 4 * m + a);
      *reinterpret_cast<half8*>(smem + off) = hi;
      *reinterpret_cast<half8*>(smem + ChunkLds<D>::KLO + off) = lo;
    }
  }
  // V: code dword (row16 = (4c + a) * 16 + i, t) holds dim 16t + i of tokens
  // 32c + 8a + 0..7; a thread takes 4 consecutive t, lanes run over i.  The
  // slab is 8 (c, a) x 16 i rows of D/4 bytes: 2D loads of 16 bytes.
  constexpr int T4 = D / 64;
  for (int ci = tid; ci < 8 * 16 * T4; ci += kCThreads) {
    const int i = ci & 15, t4 = (ci >> 4) % T4, ca = (ci >> 4) / T4;
    const int row16 = ca * 16 + i, tok0 = 8 * ca;  // 32c + 8a == 8 * (4c + a)
    const u32x4 w = *reinterpret_cast<const u32x4*>(vcs + row16 * (D / 4) + 16 * t4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int dim = 16 * (4 * t4 + k) + i, g = dim >> 5;
      const u32x4 sc = *reinterpret_cast<const u32x4*>(vss + g * 64 + tok0);
      half8 out;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float s = tok0 + e < nvalid ? half_bits(sc[e >> 1] >> (16 * (e & 1))) : 0.0f;
        out[e] = (_Float16)(lev[(w[k] >> (4 * e)) & 15] * s);
      }
      *reinterpret_cast<half8*>(smem + ChunkLds<D>::V0 + dim * VP + tok0 * 2) = out;
    }
  }
}

// ---- copy one exact block into LDS (K rows, V transposed)
template <int D>
__device__ inline void stage_exact_block(const AttnParams& p, int pb, int kv, int nvalid, unsigned char* smem) {
  constexpr int CPR = ChunkLds<D>::CPR, VP = ChunkLds<D>::VP;
  const int tid = threadIdx.x;
  const uint16_t* ks = p.ek + ((size_t)pb * p.Hkv + kv) * kBlock * D;
  const uint16_t* vs = p.ev + ((size_t)pb * p.Hkv + kv) * kBlock * D;
  for (int ci = tid; ci < 64 * CPR; ci += kCThreads) {
    const int tok = ci / CPR, ch = ci - tok * CPR;
    u32x4 kx = *reinterpret_cast<const u32x4*>(ks + tok * D + 8 * ch);
    if (tok >= nvalid) kx = u32x4{0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(smem + kchunk_off<D>(tok, ch)) = kx;
  }
  // V: a thread takes tokens 2pp, 2pp+1 of one 8-dim chunk and writes 8 dwords
  for (int ci = tid; ci < 32 * CPR; ci += kCThreads) {
    const int pp = ci & 31, ch = ci >> 5;
    u32x4 x0 = *reinterpret_cast<const u32x4*>(vs + (2 * pp) * D + 8 * ch);
    u32x4 x1 = *reinterpret_cast<const u32x4*>(vs + (2 * pp + 1) * D + 8 * ch);
    if (2 * pp >= nvalid) x0 = u32x4{0, 0, 0, 0};
    if (2 * pp + 1 >= nvalid) x1 = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t a = (x0[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      const uint32_t b = (x1[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      *reinterpret_cast<uint32_t*>(smem + ChunkLds<D>::V0 + (8 * ch + e) * VP + 4 * pp) = a | (b << 16);
    }
  }
}

// ---- one split of 128 rows
template <int D, bool QUANT>
__device__ void chunk_split(const AttnParams& p, unsigned char* smem, int b, int kv, int rg, int sx, int start,
                            int end, int el) {
  constexpr int M = D / 32, NT = D / 16, VP = ChunkLds<D>::VP;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j = lane & 15, qq = lane >> 4;
  const int G = p.G, R = p.Tq * G;
  if (QUANT && tid < 16)
    reinterpret_cast<float*>(smem + ChunkLds<D>::LEV)[tid] = __builtin_bit_cast(float, kLevelBits[tid]);

  // ---- query operands: lane (row j of tile rt, qq) holds dims 32m + 8qq + e
  const int row0 = rg * kRowsPerWG + w * 16 * kRT;
  int rowv[kRT];
  half8 Qh[kRT][M], Ql[kRT][M];
  bf16x8 Qe[kRT][M];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int r = row0 + 16 * rt + j;
    rowv[rt] = r;
    const int rr = r < R ? r : R - 1;
    const int tau = rr / G, g = rr - tau * G;
    const uint16_t* qsrc = p.q + (((size_t)b * p.Tq + tau) * p.Hq + kv * G + g) * D + 8 * qq;
    u32x4 raw[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      raw[m] = *reinterpret_cast<const u32x4*>(qsrc + 32 * m);
      if (r >= R) raw[m] = u32x4{0, 0, 0, 0};
    }
    if (QUANT) {
      float v[M][8];
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) v[m][e] = bf16_bits_to_float((raw[m][e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
      // butterflies over dim bits 0-2 (e, in lane), 3-4 (qq, across lanes), 5.. (m, in lane)
#pragma unroll
      for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (!(e & h)) {
              const float a = v[m][e], c = v[m][e + h];
              v[m][e] = a + c;
              v[m][e + h] = a - c;
            }
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float o = cxor16(v[m][e]);
          v[m][e] = (lane & 16) ? (o - v[m][e]) : (v[m][e] + o);
          o = cxor32(v[m][e]);
          v[m][e] = (lane & 32) ? (o - v[m][e]) : (v[m][e] + o);
        }
#pragma unroll
      for (int h = 1; h < M; h <<= 1)
#pragma unroll
        for (int m = 0; m < M; ++m)
          if (!(m & h))
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float a = v[m][e], c = v[m + h][e];
              v[m][e] = a + c;
              v[m + h][e] = a - c;
            }
      const float rs = inv_sqrt_d(D);
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = fp32_pinned(v[m][e] * rs * p.qscale2);
          const _Float16 hi = (_Float16)x;
          Qh[rt][m][e] = hi;
          Ql[rt][m][e] = (_Float16)(x - (float)hi);
        }
    } else {
#pragma unroll
      for (int m = 0; m < M; ++m) Qe[rt][m] = __builtin_bit_cast(bf16x8, raw[m]);
    }
  }

  float mrun[kRT], lrun[kRT];
  float4v O[NT][kRT];
  int climit[kRT];  // exact token p is visible to a row iff p <= el - Tq + tau
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    mrun[rt] = neg_inf();
    lrun[rt] = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) O[t][rt] = float4v{0, 0, 0, 0};
    climit[rt] = el - p.Tq + (rowv[rt] < R ? rowv[rt] : R - 1) / G;
  }
  const int wg_limit = el - p.Tq + (min(rg * kRowsPerWG + kRowsPerWG, R) - 1) / G;
  bool poison = false;

  const int* table = QUANT ? p.qtab + (size_t)b * p.qmax : p.etab + (size_t)b * p.emax;
  const int nbpool = QUANT ? p.qnb : p.enb;
  for (int tb = start; tb < end; tb += 64) {
    if (!QUANT && tb > wg_limit) break;  // the rest is in every row's future
    const int pb = table[tb >> 6];
    const int nvalid = min(64, end - tb);
    __syncthreads();  // every wave is done with the previous block
    if (pb < 0 || pb >= nbpool) {
      poison = true;
      continue;
    }
    if (QUANT)
      stage_quant_block<D>(p, pb, kv, nvalid, smem);
    else
      stage_exact_block<D>(p, pb, kv, nvalid, smem);
    __syncthreads();
    const bool causal_block = !QUANT && tb + 63 > el - p.Tq;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      if (tb + 32 * c >= end) break;
      // scores: row i of tile tp is token 32c + 8(i/4) + 4tp + i%4, so lane
      // (j, qq) ends up with tokens 32c + 8qq + 0..7 of row j
      float s[kRT][8];
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        const int krow = 32 * c + 8 * (j >> 2) + 4 * tp + (j & 3);
        half8 kh[M], kl[M];
        bf16x8 kb[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const int off = kchunk_off<D>(krow, 4 * m + qq);
          const u32x4 raw = *reinterpret_cast<const u32x4*>(smem + off);
          if (QUANT) {
            kh[m] = __builtin_bit_cast(half8, raw);
            kl[m] = *reinterpret_cast<const half8*>(smem + ChunkLds<D>::KLO + off);
          } else {
            kb[m] = __builtin_bit_cast(bf16x8, raw);
          }
        }
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          float4v acc = float4v{0, 0, 0, 0};
#pragma unroll
          for (int m = 0; m < M; ++m) {
            if (QUANT) {
              acc = cmfma16(kh[m], Qh[rt][m], acc);
              acc = cmfma16(kh[m], Ql[rt][m], acc);
              acc = cmfma16(kl[m], Qh[rt][m], acc);
            } else {
              acc = cmfma16bf(kb[m], Qe[rt][m], acc);
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) s[rt][4 * tp + r] = QUANT ? acc[r] : acc[r] * p.qscale2;
        }
      }
      // masks: tokens past the split end, and each row's causal future
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tok = tb + 32 * c + 8 * qq + e;
          if (tok >= end || (causal_block && tok > climit[rt])) s[rt][e] = neg_inf();
        }
      // online softmax (base 2); lanes j, j+16, j+32, j+48 share a row
      half8 ph[kRT];
      bf16x8 pbf[kRT];
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        float mx = s[rt][0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, s[rt][e]);
        mx = fmaxf(mx, cxor16(mx));
        mx = fmaxf(mx, cxor32(mx));
        const float mnew = fmaxf(mrun[rt], mx);
        const float muse = (mnew == neg_inf()) ? 0.0f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(mrun[rt] - muse);
        float sum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = __builtin_amdgcn_exp2f(s[rt][e] - muse);
          sum += pe;
          if (QUANT)
            ph[rt][e] = (_Float16)pe;
          else
            pbf[rt][e] = (__bf16)pe;
        }
        lrun[rt] = lrun[rt] * alpha + sum;
        mrun[rt] = mnew;
        if (__ballot(alpha != 1.0f)) {
#pragma unroll
          for (int t = 0; t < NT; ++t) O[t][rt] *= alpha;
        }
      }
      // values: lane (j, qq) supplies V^T[16t + j][32c + 8qq + 0..7]
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4 va =
            *reinterpret_cast<const u32x4*>(smem + ChunkLds<D>::V0 + (16 * t + j) * VP + (32 * c + 8 * qq) * 2);
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          if (QUANT)
            O[t][rt] = cmfma16(__builtin_bit_cast(half8, va), ph[rt], O[t][rt]);
          else
            O[t][rt] = cmfma16bf(__builtin_bit_cast(bf16x8, va), pbf[rt], O[t][rt]);
        }
      }
    }
  }

  // ---- partial rows straight from registers: lane holds O^T[16t + 4qq + r][row j]
  const size_t S = (size_t)p.Sq + p.Se;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int r = rowv[rt];
    float l = lrun[rt];
    l += cxor16(l);
    l += cxor32(l);
    if (r >= R) continue;
    const size_t prow = ((size_t)(b * p.Hkv + kv) * S + sx) * R + r;
    float* dst = p.part_o + prow * D;
    const bool empty = mrun[rt] == neg_inf();
    const float inv = empty ? 0.0f : 1.0f / l;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float4v v = O[t][rt] * inv;
      if (poison) v = float4v{1, 1, 1, 1} * __builtin_nanf("");
      *reinterpret_cast<float4v*>(dst + 16 * t + 4 * qq) = v;
    }
    if (qq == 0)
      p.part_lse[prow] = poison ? __builtin_nanf("") : (empty ? neg_inf() : (mrun[rt] + __builtin_log2f(l)) * kLn2);
  }
}

// grid (Hkv * nrg, Sq + Se, B): the long compressed-tier splits come first in
// dispatch order, the shorter exact-tier splits fill in behind them.
template <int D>
__global__ __launch_bounds__(kCThreads, 2) void chunk_split_kernel(AttnParams p, int nrg) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[ChunkLds<D>::BYTES];
  const int kv = blockIdx.x / nrg, rg = blockIdx.x - kv * nrg, sx = blockIdx.y, b = blockIdx.z;
  const int ql = p.qmax ? p.qlen[b] : 0;
  const int el = p.emax ? p.elen[b] : 0;
  if (ql < 0 || ql > p.qmax * 64 || el < p.Tq || el > p.emax * 64) return;  // merge writes NaN
  const bool quant = sx < p.Sq;
  const int s = quant ? sx : sx - p.Sq;
  const int P = quant ? p.Pq : p.Pe;
  const int len = quant ? ql : el;
  const int start = s * P;
  if (start >= len) return;
  const int end = min(start + P, len);
  if (quant)
    chunk_split<D, true>(p, smem, b, kv, rg, sx, start, end, el);
  else
    chunk_split<D, false>(p, smem, b, kv, rg, sx, start, end, el);
}

// ---- merge: one wave per (sequence, query token, query head)
template <int D>
__global__ __launch_bounds__(256) void chunk_merge_kernel(AttnParams p) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int rowq = blockIdx.x * 4 + (threadIdx.x >> 6), b = blockIdx.y;
  if (rowq >= p.Tq * p.Hq) return;
  const int tau = rowq / p.Hq, h = rowq - tau * p.Hq;
  const int G = p.G, kv = h / G, g = h - kv * G, R = p.Tq * G;
  float* out = p.o + (((size_t)b * p.Tq + tau) * p.Hq + h) * D;
  float* lout = p.lse + ((size_t)b * p.Tq + tau) * p.Hq + h;
  const int ql = p.qmax ? p.qlen[b] : 0;
  const int el = p.emax ? p.elen[b] : 0;
  if (ql < 0 || ql > 64 * p.qmax || el < p.Tq || el > 64 * p.emax) {
#pragma unroll
    for (int e = 0; e < E; ++e) out[lane + 64 * e] = __builtin_nanf("");
    if (lane == 0) *lout = __builtin_nanf("");
    return;
  }
  const int nq = (ql + p.Pq - 1) / p.Pq, ne = (el + p.Pe - 1) / p.Pe;
  const size_t S = (size_t)p.Sq + p.Se;
  const size_t base = ((size_t)(b * p.Hkv + kv) * S) * R + tau * G + g;
  float res_o[2][E], res_l[2];
#pragma unroll
  for (int tier = 0; tier < 2; ++tier) {
    const int n = tier ? ne : nq;
    const size_t first = base + (tier ? (size_t)p.Sq * R : 0);
    float m = neg_inf(), wsum = 0.0f;
    float acc[E];
    bool nan = false;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;
    for (int s = 0; s < n; ++s) {
      const size_t r = first + (size_t)s * R;
      const float l = p.part_lse[r];
      float x[E];
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = p.part_o[r * D + lane + 64 * e];
      if (l != l) {
        nan = true;
        continue;
      }
      if (l == neg_inf()) continue;
      if (l > m) {
        const float f = (m == neg_inf()) ? 0.0f : __expf(m - l);
        wsum *= f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] *= f;
        m = l;
      }
      const float wt = __expf(l - m);
      wsum += wt;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += wt * x[e];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) res_o[tier][e] = (m == neg_inf()) ? 0.0f : acc[e] / wsum;
    res_l[tier] = nan ? __builtin_nanf("") : (m == neg_inf() ? neg_inf() : m + __logf(wsum));
  }
  // inverse rotation of the compressed-tier output: dim = lane + 64e
#pragma unroll
  for (int hh = 1; hh < 64; hh <<= 1)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float o = __shfl_xor(res_o[0][e], hh);
      res_o[0][e] = (lane & hh) ? (o - res_o[0][e]) : (res_o[0][e] + o);
    }
  if constexpr (E == 2) {
    const float a = res_o[0][0], c = res_o[0][1];
    res_o[0][0] = a + c;
    res_o[0][1] = a - c;
  }
  const float rd = inv_sqrt_d(D);
  const float la = res_l[0], lb = res_l[1];
  const bool bad = la != la || lb != lb;
  const float Mx = fmaxf(la, lb);
  const bool none = !bad && Mx == neg_inf();
  const float wa = (bad || none) ? 0.0f : __expf(la - Mx), wb = (bad || none) ? 0.0f : __expf(lb - Mx);
  const float W = wa + wb;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float o;
    if (bad)
      o = __builtin_nanf("");
    else if (none)
      o = 0.0f;
    else
      o = (wa / W) * (res_o[0][e] * rd) + (wb / W) * res_o[1][e];
    out[lane + 64 * e] = o;
  }
  if (lane == 0) *lout = bad ? __builtin_nanf("") : (none ? neg_inf() : Mx + __logf(W));
}

hipError_t launch_chunk(const AttnParams& p, int D, hipStream_t stream) {
  const int R = p.Tq * p.G;
  const int nrg = (R + kRowsPerWG - 1) / kRowsPerWG;
  const dim3 grid(p.Hkv * nrg, p.Sq + p.Se, p.B);
  const dim3 mgrid((p.Tq * p.Hq + 3) / 4, p.B);
  if (D == 64) {
    hipLaunchKernelGGL(chunk_split_kernel<64>, grid, dim3(kCThreads), 0, stream, p, nrg);
    hipLaunchKernelGGL(chunk_merge_kernel<64>, mgrid, dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(chunk_split_kernel<128>, grid, dim3(kCThreads), 0, stream, p, nrg);
    hipLaunchKernelGGL(chunk_merge_kernel<128>, mgrid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace akv
