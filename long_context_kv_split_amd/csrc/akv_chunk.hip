// Prefill-chunk attention: Tq causal queries per sequence over the two-tier
// history, on 16x16x32 matrix-core tiles (ActiveKV, "Context beyond VRAM",
// "What I built": a full-precision recent window and an encoded older tier,
// combined without approximation; the encoded tier is read through the
// pre-rotated query of the QuantForge walkthrough, section 1).
//
// Rows of one kv head are (query, head) pairs r = tau * G + g.  A workgroup
// (4 waves x 32 rows; two workgroups per CU) takes
// 128 consecutive rows and one split (a run of whole blocks of one tier).
// Each 64-token block is expanded once into LDS and used by all 128 rows:
//   compressed tier: K[token][dim] = C[code] * scale in fp32, stored as fp16
//     hi + lo parts, and the transposed V^T[dim][token] = fp16(C16[code] x
//     scale) (packed fp16 product).  The query is rotated by the Walsh-
//     Hadamard butterflies in fp32 and split into fp16 hi + lo parts; a score
//     is Khi.Qhi + Khi.Qlo + Klo.Qhi (three tiles), about 22 significant
//     bits, so the log-sum-exp keeps fp32-like accuracy on short or
//     outlier-heavy histories;
//   exact tier: bf16 K rows and transposed bf16 V with the bf16 query (exact
//     products, fp32 sums); the last Tq exact tokens are the chunk itself and
//     query tau sees chunk tokens <= tau.
// Per wave:  S^T[token][row] = K_tile x Q^T  and  O^T[dim][row] += V^T x P^T,
// with an online softmax per row.
// Pipeline: one LDS block buffer per workgroup (two workgroups share a CU)
// and one register set: a block is expanded from registers into LDS, the
// next block is requested from HBM into the registers, and the block is
// computed while those loads are in flight.
// Every wave owns its rows, so a split's partial (normalized output,
// log-sum-exp) is written straight from registers.  A second kernel merges
// each row's splits in ascending order: compressed-tier splits in rotated
// space, one inverse rotation, exact-tier splits, then both tiers.
// Variants (compile-time, so the 4-bit Walsh-Hadamard kernels are unchanged):
// a caller-given rotation R (the query is rotated by R in a small kernel
// before the splits and the merge applies R^T in place of the butterflies),
// and code widths 2 and 3 (the narrow planes are turned into the same
// two-code table fields, with 4^W-entry tables).
#include "akv_common.h"
#include "akv_params.h"

namespace akv {

constexpr int kCWaves = 4;
constexpr int kCThreads = 64 * kCWaves;
constexpr int kRT = 2;                       // 16-row tiles per wave
constexpr int kVT = 512 / kCThreads;         // staging slots (of 512 per block) per thread
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
// the hi that lo was taken from differ by one ulp.  The empty asm is not
// volatile: it hides the value without ordering the conversions of one
// staged block against each other.
__device__ inline float fp32_pinned(float x) {
  asm("" : "+v"(x));
  return x;
}

// LDS layout: two byte tables, then the block buffer (K hi rows, K lo rows,
// V^T rows), rows unpadded.  A 128-bit LDS access on gfx950 serves 16 lanes
// per cycle over 64 banks, in lane groups that are not simply 16 consecutive
// lanes, so the chunk permutations below were chosen by measuring the bank-
// conflict counter for the operand reads and the staging writes (all zero):
//   K row t:     16-byte chunk c at position c ^ ((t & 3) | ((t >> 3) & 3) << 2);
//   V^T row dim: 16-byte chunk c (8 tokens) at position c ^ (dim & 7).
template <int D>
struct ChunkLds {
  static constexpr int CPR = D / 8;            // 16-byte chunks per K row
  static constexpr int KP = D * 2;
  static constexpr int VP = 64 * 2;
  static constexpr int K_BYTES = 64 * KP;
  static constexpr int KLO = K_BYTES;          // compressed tier: K lo parts (buffer-relative)
  static constexpr int V0 = 2 * K_BYTES;       // V^T rows (buffer-relative)
  static constexpr int BUF = V0 + D * VP;
  static constexpr int KLUT = 0;               // 256 x (level lo nibble, level hi nibble) fp32
  static constexpr int VLUT = 256 * 8;         // 256 x the same in fp16
  static constexpr int BUF0 = VLUT + 256 * 4;  // the block buffer
  static constexpr int BYTES = BUF0 + BUF;
};

template <int D>
__device__ inline int kchunk_off(int t, int c) {
  const int h = ((t & 3) | (((t >> 3) & 3) << 2)) & (ChunkLds<D>::CPR - 1);
  return t * ChunkLds<D>::KP + 16 * (c ^ h);
}
// byte offset of tokens 8c .. 8c + 7 of V^T row dim
template <int D>
__device__ inline int vchunk_off(int dim, int c) {
  return ChunkLds<D>::V0 + dim * ChunkLds<D>::VP + 16 * (c ^ (dim & 7));
}

// ---------------------------------------------------------------- staging
// Register copy of one block's share for this thread.
// A block's staging work is cut into 512 slots; thread t takes slots
// t + kCThreads * u (u < kVT).
// W: code width.  At W = 4 a code dword holds four table fields (bytes, two
// codes each); at W = 2 and 3 it is the pair-plane dword whose nibbles
// (at W = 3 with two high-plane bits above each) form the fields.
template <int D, int W>
struct QRegs {
  static constexpr int KDW = D / 64;  // K code dwords per slot
  static constexpr int VDW = D / 64;  // V code dwords per slot
  uint32_t kc[kVT][KDW];
  uint32_t kh[kVT][KDW];  // W = 3: the high-plane bits of the slot's K dims
  uint32_t ks[kVT][KDW];  // fp16 K scale of each dword's group (low 16 bits)
  uint32_t vc[kVT][VDW];
  uint32_t vh[kVT][VDW];  // W = 3: the high-plane bits of the slot's V tiles
  u32x4 vs[kVT];          // fp16 V scales of the slot's group, tokens tok0 .. tok0 + 7
};

// Table fields of K dword k of slot u (group m, dims 32m + 8a + 2b, +1 in
// byte b) and of V dword k (value tile tt).
template <int D, int W>
__device__ inline uint32_t chunk_kfield(const QRegs<D, W>& r, int u, int k, int m) {
  if constexpr (W == 4) {
    return r.kc[u][k];
  } else {
    uint32_t f = (r.kc[u][k] >> (4 * (m & 1))) & 0x0F0F0F0Fu;
    if constexpr (W == 3) f |= ((r.kh[u][k] >> (2 * m)) & 0x03030303u) << 4;
    return f;
  }
}
template <int D, int W>
__device__ inline uint32_t chunk_vfield(const QRegs<D, W>& r, int u, int k, int tt) {
  if constexpr (W == 4) {
    return r.vc[u][k];
  } else {
    uint32_t f = (r.vc[u][k] >> (4 * (tt & 1))) & 0x0F0F0F0Fu;
    if constexpr (W == 3) f |= ((r.vh[u][k] >> (2 * (tt & 3))) & 0x03030303u) << 4;
    return f;
  }
}
template <int D>
struct ERegs {
  static constexpr int KCH = 64 * D / 8 / 512;  // 16-byte K chunks per slot
  u32x4 k[kVT][KCH];
  u32x4 v[kVT][D / 64];    // 16-byte V chunks v + 512 h: dim (v + 512 h) / 8, tokens 8 ((v + 512 h) % 8) ..
};

// Slot v's K dwords: token v / 8, dword wi_k = 4 (p & 3) + (p >> 2) + 2k of
// the row (p = v % 8; D = 128), which holds dims 32 (wi % M) + 8 (wi / M) + 0..7.
template <int D>
__device__ inline int qk_dword(int t, int k) {
  if constexpr (D == 128) {
    const int p = t & 7;
    return 4 * (p & 3) + (p >> 2) + 2 * k;
  } else {
    return t & 7;
  }
}

template <int D, int W>
__device__ inline void quant_fetch(QRegs<D, W>& r, const AttnParams& p, int pb, int kv) {
  constexpr int M = D / 32;
  const int t = threadIdx.x;
  const size_t slab = (size_t)pb * p.Hkv + kv;
  const uint32_t* kcs = reinterpret_cast<const uint32_t*>(p.kc + slab * (8 * W * D));
  const uint32_t* vcs = reinterpret_cast<const uint32_t*>(p.vc + slab * (8 * W * D));
  const uint16_t* kss = p.ks + slab * (2 * D);
  const uint16_t* vss = p.vs + slab * (2 * D);
#pragma unroll
  for (int u = 0; u < kVT; ++u) {
    const int v = t + kCThreads * u, tok = v >> 3;
#pragma unroll
    for (int k = 0; k < QRegs<D, W>::KDW; ++k) {
      const int wi = qk_dword<D>(v, k), m = wi % M, a = wi / M;
      if constexpr (W == 4) {
        r.kc[u][k] = kcs[tok * (D / 8) + wi];
      } else {
        // pair plane: token rows of D/4 bytes, dword (D/64) a + m/2 holds
        // groups m & ~1 and m | 1 in its low and high nibbles
        r.kc[u][k] = kcs[tok * (D / 16) + (D / 64) * a + (m >> 1)];
        if constexpr (W == 3) {
          // high plane after the pair plane: token rows of D/8 bytes; the
          // two bits of dims 32m + 8a + 2b, +1 at row bit 8 M a + 2 M b + 2m
          const unsigned char* hrow = reinterpret_cast<const unsigned char*>(kcs) + 16 * D + tok * (D / 8);
          if constexpr (D == 128) {
            r.kh[u][k] = reinterpret_cast<const uint32_t*>(hrow)[a];
          } else {  // 16 bits per a: nibble b -> byte b
            const uint32_t h = reinterpret_cast<const uint16_t*>(hrow)[a];
            r.kh[u][k] = (h & 0xFu) | ((h << 4) & 0xF00u) | ((h << 8) & 0xF0000u) | ((h << 12) & 0xF000000u);
          }
        }
      }
      r.ks[u][k] = kss[m * 64 + tok];
    }
    // V: slots run over i (dim within 16), then over 4 dword columns, then 8
    // token groups (c, a); dword of tile t at c*16D + (t/4)*1 KB + (16a + i)*16 + 4(t%4) bytes
    const int i = v & 15, tq = (v >> 4) & 3, ca = v >> 6;
#pragma unroll
    for (int k = 0; k < QRegs<D, W>::VDW; ++k) {
      const int tt = tq * QRegs<D, W>::VDW + k;
      if constexpr (W == 4) {
        r.vc[u][k] = vcs[(ca >> 2) * 4 * D + (tt >> 2) * 256 + ((ca & 3) * 16 + i) * 4 + (tt & 3)];
      } else {
        // pair plane: D/8 bytes per (token group ca, lane dim i), dword tt/2
        // holds tiles tt & ~1 and tt | 1 in its low and high nibbles
        r.vc[u][k] = vcs[(ca * 16 + i) * (D / 32) + (tt >> 1)];
        if constexpr (W == 3)  // high plane: D/16 bytes per (ca, i), dword tt/4, bits 2 (tt % 4) of each byte
          r.vh[u][k] = reinterpret_cast<const uint32_t*>(reinterpret_cast<const unsigned char*>(vcs) + 16 * D)
              [(ca * 16 + i) * (D / 64) + (tt >> 2)];
      }
    }
    const int g = (16 * tq * QRegs<D, W>::VDW + i) >> 5;
    r.vs[u] = *reinterpret_cast<const u32x4*>(vss + g * 64 + 8 * ca);
  }
}

template <int D>
__device__ inline void exact_fetch(ERegs<D>& r, const AttnParams& p, int pb, int kv) {
  constexpr int CPR = ChunkLds<D>::CPR;
  const int t = threadIdx.x;
  const uint16_t* ks = p.ek + ((size_t)pb * p.Hkv + kv) * kBlock * D;
  const uint16_t* vs = p.ev + ((size_t)pb * p.Hkv + kv) * kBlock * D;
#pragma unroll
  for (int u = 0; u < kVT; ++u) {
    const int v = t + kCThreads * u;
#pragma unroll
    for (int k = 0; k < ERegs<D>::KCH; ++k) {
      const int ci = v + 512 * k, tok = ci / CPR, ch = ci - tok * CPR;
      r.k[u][k] = *reinterpret_cast<const u32x4*>(ks + tok * D + 8 * ch);
    }
    // V is dim-major inside each half block: chunk c8 of dim t (tokens
    // 8 c8 ..) sits in half c8 / 4, at ((c8 / 4) * D + t) * 32 + 8 (c8 % 4)
#pragma unroll
    for (int h = 0; h < D / 64; ++h) {
      const int ci = v + 512 * h, c8 = ci & 7;
      r.v[u][h] = *reinterpret_cast<const u32x4*>(vs + ((c8 >> 2) * D + (ci >> 3)) * (kBlock / 2) + 8 * (c8 & 3));
    }
  }
}

// Compressed K -> LDS (fp16 hi + lo of the fp32 product level x scale).
template <int D, int W>
__device__ inline void quant_stage_k(const QRegs<D, W>& r, unsigned char* smem, unsigned char* buf, int nvalid) {
  constexpr int M = D / 32;
  const float2* klut = reinterpret_cast<const float2*>(smem + ChunkLds<D>::KLUT);
  // every table read of this thread's share first, so they are in flight
  // together, then the products and conversions
  float2 lvs[kVT][QRegs<D, W>::KDW][4];
#pragma unroll
  for (int u = 0; u < kVT; ++u)
#pragma unroll
    for (int k = 0; k < QRegs<D, W>::KDW; ++k) {
      const uint32_t f = chunk_kfield<D, W>(r, u, k, qk_dword<D>(threadIdx.x + kCThreads * u, k) % M);
#pragma unroll
      for (int b = 0; b < 4; ++b) lvs[u][k][b] = klut[(f >> (8 * b)) & 0xFFu];
    }
#pragma unroll
  for (int u = 0; u < kVT; ++u)
#pragma unroll
  for (int k = 0; k < QRegs<D, W>::KDW; ++k) {
    const int v = threadIdx.x + kCThreads * u, tok = v >> 3;
    const int wi = qk_dword<D>(v, k), m = wi % M, a = wi / M;
    const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(tok < nvalid ? r.ks[u][k] & 0xFFFFu : 0u));
    half8 hi, lo;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float2 lv = lvs[u][k][b];
      // hi = fp16(c s) and lo = fp16(c s - hi), each one rounding of an exact
      // fused product (mixed-precision FMAs)
      hi[2 * b] = (_Float16)__builtin_fmaf(lv.x, s, 0.0f);
      hi[2 * b + 1] = (_Float16)__builtin_fmaf(lv.y, s, 0.0f);
      lo[2 * b] = (_Float16)__builtin_fmaf(lv.x, s, -(float)hi[2 * b]);
      lo[2 * b + 1] = (_Float16)__builtin_fmaf(lv.y, s, -(float)hi[2 * b + 1]);
    }
    const int off = kchunk_off<D>(tok, 4 * m + a);
    *reinterpret_cast<half8*>(buf + off) = hi;
    *reinterpret_cast<half8*>(buf + ChunkLds<D>::KLO + off) = lo;
  }
}

// Compressed V -> LDS as V^T (fp16 level pair x fp16 scale pair).
template <int D, int W>
__device__ inline void quant_stage_v(const QRegs<D, W>& r, unsigned char* smem, unsigned char* buf, int nvalid) {
  const uint32_t* vlut = reinterpret_cast<const uint32_t*>(smem + ChunkLds<D>::VLUT);
#pragma unroll
  for (int u = 0; u < kVT; ++u) {
    const int v = threadIdx.x + kCThreads * u, i = v & 15, tq = (v >> 4) & 3, ca = v >> 6, tok0 = 8 * ca;
    u32x4 sc = r.vs[u];
    if (nvalid < 64 && tok0 + 8 > nvalid) {  // nvalid is the block's: only its last block masks
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (tok0 + 2 * b >= nvalid) sc[b] = 0u;
        else if (tok0 + 2 * b + 1 >= nvalid) sc[b] &= 0xFFFFu;
      }
    }
#pragma unroll
    for (int k = 0; k < QRegs<D, W>::VDW; ++k) {
      const int tt = tq * QRegs<D, W>::VDW + k, dim = 16 * tt + i;
      const uint32_t f = chunk_vfield<D, W>(r, u, k, tt);
      u32x4 out;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const half2v lv = __builtin_bit_cast(half2v, vlut[(f >> (8 * b)) & 0xFFu]);
        // copy the element out first: a bit cast applied to a vector element
        // expression reads element 0 whatever the index
        const uint32_t sb = sc[b];
        out[b] = __builtin_bit_cast(uint32_t, lv * __builtin_bit_cast(half2v, sb));
      }
      *reinterpret_cast<u32x4*>(buf + vchunk_off<D>(dim, ca)) = out;
    }
  }
}

template <int D>
__device__ inline void exact_stage_k(const ERegs<D>& r, unsigned char* buf, int nvalid) {
  constexpr int CPR = ChunkLds<D>::CPR;
#pragma unroll
  for (int u = 0; u < kVT; ++u)
#pragma unroll
  for (int k = 0; k < ERegs<D>::KCH; ++k) {
    const int ci = threadIdx.x + kCThreads * u + 512 * k, tok = ci / CPR, ch = ci - tok * CPR;
    const u32x4 x = tok < nvalid ? r.k[u][k] : u32x4{0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(buf + kchunk_off<D>(tok, ch)) = x;
  }
}

template <int D>
__device__ inline void exact_stage_v(const ERegs<D>& r, unsigned char* buf, int nvalid) {
#pragma unroll
  for (int u = 0; u < kVT; ++u) {
    const int v = threadIdx.x + kCThreads * u;
#pragma unroll
    for (int h = 0; h < D / 64; ++h) {
      const int ci = v + 512 * h, dim = ci >> 3, c = ci & 7;
      u32x4 x = r.v[u][h];
      if (nvalid < 64) {  // zero tokens 8c + 2i (low half), 8c + 2i + 1 (high half) past the length
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t0 = 8 * c + 2 * i;
          x[i] &= t0 >= nvalid ? 0u : (t0 + 1 >= nvalid ? 0xFFFFu : ~0u);
        }
      }
      *reinterpret_cast<u32x4*>(buf + vchunk_off<D>(dim, c)) = x;
    }
  }
}

// ---------------------------------------------------------------- compute
// Online softmax in base 2 against a reference m per row: l and O hold sums
// of 2^(s - m), and moving m rescales them; the log-sum-exp m + log2 l and
// O / l do not depend on where m sits.  The compressed tier moves m up to the
// row maximum only when a score exceeds it by more than kLazyShift (an fp16
// probability is then at most 2^8).  The exact tier's probabilities are
// rounded to bf16 (8 significant bits) before the product with V while l sums
// them unrounded, so it moves m whenever a score exceeds it: the row
// maximum's probability stays exactly 1 and the dominant term is not rounded.
constexpr float kLazyShift = 8.0f;

template <int D>
struct RowState {
  float m[kRT], l[kRT];  // m = -inf until the row has seen a score
  float4v O[D / 16][kRT];
};

// One 32-token half (c) of a staged block for this wave's 32 rows.
// mask: apply the split end and the causal limits (last block / chunk blocks).
template <int D, bool QUANT>
__device__ inline void compute_half(const unsigned char* buf, int c, bool mask, int tb, int end, const int (&climit)[kRT],
                                    const half8 (&Qh)[kRT][D / 32], const half8 (&Ql)[kRT][D / 32],
                                    const bf16x8 (&Qe)[kRT][D / 32], float qs, RowState<D>& rs) {
  constexpr int M = D / 32, NT = D / 16;
  const int lane = threadIdx.x & 63, j = lane & 15, qq = lane >> 4;
  // scores relative to the reference: s - base, base = m (0 before any score)
  float base[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) base[rt] = rs.m[rt] == neg_inf() ? 0.0f : rs.m[rt];
  // scores: row i of tile tp is token 32c + 8(i/4) + 4tp + i%4, so lane
  // (j, qq) ends up with tokens 32c + 8qq + 0..7 of row j
  float s[kRT][8];
  // key operands of both 16-token tiles read up front, so the second tile's
  // reads are in flight while the first tile's products run
  half8 kh[2][M], kl[2][M];
  bf16x8 kb[2][M];
#pragma unroll
  for (int tp = 0; tp < 2; ++tp) {
    const int krow = 32 * c + 8 * (j >> 2) + 4 * tp + (j & 3);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int off = kchunk_off<D>(krow, 4 * m + qq);
      const u32x4 raw = *reinterpret_cast<const u32x4*>(buf + off);
      if (QUANT) {
        kh[tp][m] = __builtin_bit_cast(half8, raw);
        kl[tp][m] = *reinterpret_cast<const half8*>(buf + ChunkLds<D>::KLO + off);
      } else {
        kb[tp][m] = __builtin_bit_cast(bf16x8, raw);
      }
    }
  }
#pragma unroll
  for (int tp = 0; tp < 2; ++tp) {
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      // the compressed tier's query carries the score scale, so the tile
      // starts from -base; the exact tier scales afterwards
      const float a0 = QUANT ? -base[rt] : 0.0f;
      float4v acc = float4v{a0, a0, a0, a0};
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if (QUANT) {
          acc = cmfma16(kh[tp][m], Qh[rt][m], acc);
          acc = cmfma16(kh[tp][m], Ql[rt][m], acc);
          acc = cmfma16(kl[tp][m], Qh[rt][m], acc);
        } else {
          acc = cmfma16bf(kb[tp][m], Qe[rt][m], acc);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) s[rt][4 * tp + r] = QUANT ? acc[r] : __builtin_fmaf(acc[r], qs, -base[rt]);
    }
  }
  // value operands: lane (j, qq) supplies V^T[16t + j][32c + 8qq + 0..7];
  // read before the softmax, which does not need them, so the reads are in
  // flight while it runs
  u32x4 va[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) va[t] = *reinterpret_cast<const u32x4*>(buf + vchunk_off<D>(16 * t + j, 4 * c + qq));
  if (mask) {
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = tb + 32 * c + 8 * qq + e;
        if (tok >= end || tok > climit[rt]) s[rt][e] = neg_inf();
      }
  }
  // online softmax; lanes j, j+16, j+32, j+48 share a row.  The reference
  // moves (for the whole wave at once) when a row has no reference yet or a
  // score exceeds it by more than the tier's allowance; a NaN score also
  // takes that path and ends as a NaN output.
  constexpr float lazy = QUANT ? kLazyShift : 0.0f;
  bool move = false;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    float mx = s[rt][0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, s[rt][e]);
    move |= !(mx <= lazy) || rs.m[rt] == neg_inf();
  }
  if (__ballot(move)) {
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      float mx = s[rt][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, s[rt][e]);
      mx = fmaxf(mx, cxor16(mx));
      mx = fmaxf(mx, cxor32(mx));
      // shift d of the reference: to the row maximum, never down once set
      const bool fresh = rs.m[rt] == neg_inf();
      const float d = fresh ? (mx == neg_inf() ? 0.0f : mx) : fmaxf(mx, 0.0f);
      if (!(fresh && mx == neg_inf())) rs.m[rt] = base[rt] + d;
      const float alpha = fresh ? 1.0f : __builtin_amdgcn_exp2f(-d);  // O and l are 0 while fresh
#pragma unroll
      for (int e = 0; e < 8; ++e) s[rt][e] -= d;
      rs.l[rt] *= alpha;
      if (__ballot(alpha != 1.0f)) {
#pragma unroll
        for (int t = 0; t < NT; ++t) rs.O[t][rt] *= alpha;
      }
    }
  }
  half8 ph[kRT];
  bf16x8 pbf[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    float sum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = __builtin_amdgcn_exp2f(s[rt][e]);
      sum += pe;
      if (QUANT)
        ph[rt][e] = (_Float16)pe;
      else
        pbf[rt][e] = (__bf16)pe;
    }
    rs.l[rt] += sum;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      if (QUANT)
        rs.O[t][rt] = cmfma16(__builtin_bit_cast(half8, va[t]), ph[rt], rs.O[t][rt]);
      else
        rs.O[t][rt] = cmfma16bf(__builtin_bit_cast(bf16x8, va[t]), pbf[rt], rs.O[t][rt]);
    }
  }
}

// ---------------------------------------------------------------- one split
template <int D, bool QUANT, bool ROT, int W>
__device__ void chunk_split(const AttnParams& p, unsigned char* smem, int b, int kv, int rg, int sx, int start,
                            int end, int el) {
  constexpr int M = D / 32, NT = D / 16;
  using Regs = typename std::conditional<QUANT, QRegs<D, W>, ERegs<D>>::type;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j = lane & 15, qq = lane >> 4;
  const int G = p.G, R = p.Tq * G;

  // ---- blocks of this split (the exact tier stops at the last block any row sees)
  int nb = ((end + 63) >> 6) - (start >> 6);
  if (!QUANT) {
    const int wg_limit = el - p.Tq + (min(rg * kRowsPerWG + kRowsPerWG, R) - 1) / G;
    nb = min(nb, wg_limit < start ? 0 : ((wg_limit - start) >> 6) + 1);
  }
  const int* table = QUANT ? p.qtab + (size_t)b * p.qmax : p.etab + (size_t)b * p.emax;
  const int nbpool = QUANT ? p.qnb : p.enb;
  bool poison = false;
  // pool block of raw table entry pb (a bad id poisons the split and reads block 0)
  auto checked = [&](int pb) {
    const bool ok = pb >= 0 && pb < nbpool;
    poison |= !ok;
    return ok ? pb : 0;
  };
  auto raw_id = [&](int n) { return n < nb ? table[(start >> 6) + n] : 0; };
  auto fetch = [&](Regs& r, int pb) {
    if constexpr (QUANT)
      quant_fetch<D, W>(r, p, checked(pb), kv);
    else
      exact_fetch<D>(r, p, checked(pb), kv);
  };

  // ---- field tables (compressed tier): entry e holds the levels of the two
  // codes of field e (W = 4: nibbles; W = 2: 2-bit halves; W = 3: 2-bit
  // halves with their top bits in bits 4 and 5)
  for (int e = tid; QUANT && e < (1 << (2 * W)); e += kCThreads) {
    int i0, i1;
    if constexpr (W == 4) {
      i0 = e & 15, i1 = e >> 4;
    } else if constexpr (W == 3) {
      i0 = (e & 3) | (((e >> 4) & 1) << 2), i1 = ((e >> 2) & 3) | (((e >> 5) & 1) << 2);
    } else {
      i0 = e & 3, i1 = (e >> 2) & 3;
    }
    const float c0 = __builtin_bit_cast(float, level_bits<W>()[i0]);
    const float c1 = __builtin_bit_cast(float, level_bits<W>()[i1]);
    reinterpret_cast<float2*>(smem + ChunkLds<D>::KLUT)[e] = float2{c0, c1};
    reinterpret_cast<half2v*>(smem + ChunkLds<D>::VLUT)[e] = half2v{(_Float16)c0, (_Float16)c1};
  }

  // ---- query operands: lane (row j of tile rt, qq) holds dims 32m + 8qq + e
  const int row0 = rg * kRowsPerWG + w * 16 * kRT;
  int rowv[kRT], climit[kRT];
  half8 Qh[kRT][M], Ql[kRT][M];
  bf16x8 Qe[kRT][M];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int r = row0 + 16 * rt + j;
    rowv[rt] = r;
    const int rr = r < R ? r : R - 1;
    const int tau = rr / G, g = rr - tau * G;
    climit[rt] = QUANT ? 0x7FFFFFFF : el - p.Tq + tau;  // exact token p is visible iff p <= el - Tq + tau
    const uint16_t* qsrc = p.q + (((size_t)b * p.Tq + tau) * p.Hq + kv * G + g) * D + 8 * qq;
    u32x4 raw[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      raw[m] = *reinterpret_cast<const u32x4*>(qsrc + 32 * m);
      if (r >= R) raw[m] = u32x4{0, 0, 0, 0};
    }
    if constexpr (QUANT && ROT) {
      // a given rotation R: R q was formed once per call (qrot_kernel); the
      // compressed tier is read through it as it is
      const float* qr = p.qrot + (((size_t)b * p.Tq + tau) * p.Hq + kv * G + g) * D + 8 * qq;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float4v a = *reinterpret_cast<const float4v*>(qr + 32 * m);
        float4v c = *reinterpret_cast<const float4v*>(qr + 32 * m + 4);
        if (r >= R) a = c = float4v{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = fp32_pinned((e < 4 ? a[e] : c[e - 4]) * p.qscale2);
          const _Float16 hi = (_Float16)x;
          Qh[rt][m][e] = hi;
          Ql[rt][m][e] = (_Float16)(x - (float)hi);
        }
      }
    } else if constexpr (QUANT) {
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

  RowState<D> rs;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    rs.m[rt] = neg_inf();
    rs.l[rt] = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) rs.O[t][rt] = float4v{0, 0, 0, 0};
  }

  unsigned char* buf = smem + ChunkLds<D>::BUF0;
  auto nvalid_of = [&](int n) { return min(64, end - (start + 64 * n)); };
  const int causal_from = el - p.Tq;  // blocks reaching past this token need the causal mask
  Regs regs;
  // block ids are read one block ahead of their fetch, so a fetch does not
  // wait for its table entry
  if (nb > 0) fetch(regs, raw_id(0));
  int id_next = raw_id(1);
  __syncthreads();  // byte tables visible
  for (int n = 0; n < nb; ++n) {
    if (n) __syncthreads();  // every wave is done with the previous block
    if constexpr (QUANT) {
      quant_stage_k<D, W>(regs, smem, buf, nvalid_of(n));
      quant_stage_v<D, W>(regs, smem, buf, nvalid_of(n));
    } else {
      exact_stage_k<D>(regs, buf, nvalid_of(n));
      exact_stage_v<D>(regs, buf, nvalid_of(n));
    }
    __syncthreads();
    if (n + 1 < nb) {  // in flight while this block is computed
      const int id2 = raw_id(n + 2);
      fetch(regs, id_next);
      id_next = id2;
    }
    const int tb = start + 64 * n;
    const bool mask = (tb + 64 > end) || (!QUANT && tb + 63 > causal_from);
    compute_half<D, QUANT>(buf, 0, mask, tb, end, climit, Qh, Ql, Qe, p.qscale2, rs);
    if (tb + 32 < end) compute_half<D, QUANT>(buf, 1, mask, tb, end, climit, Qh, Ql, Qe, p.qscale2, rs);
  }

  // ---- partial rows straight from registers: lane holds O^T[16t + 4qq + r][row j]
  const size_t S = (size_t)p.Sq + p.Se;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int r = rowv[rt];
    float l = rs.l[rt];
    l += cxor16(l);
    l += cxor32(l);
    if (r >= R) continue;
    const size_t prow = ((size_t)(b * p.Hkv + kv) * S + sx) * R + r;
    float* dst = p.part_o + prow * D;
    const bool empty = rs.m[rt] == neg_inf();
    const float inv = empty ? 0.0f : 1.0f / l;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float4v v = rs.O[t][rt] * inv;
      if (poison) v = float4v{1, 1, 1, 1} * __builtin_nanf("");
      *reinterpret_cast<float4v*>(dst + 16 * t + 4 * qq) = v;
    }
    if (qq == 0)
      p.part_lse[prow] = poison ? __builtin_nanf("") : (empty ? neg_inf() : (rs.m[rt] + __builtin_log2f(l)) * kLn2);
  }
}

// grid (Hkv * nrg, Sq + Se, B): the long compressed-tier splits come first in
// dispatch order, the shorter exact-tier splits fill in behind them.  At
// d = 64 three workgroups share a compute unit (168 VGPRs, a few spilled,
// and 27 KB of LDS each), at d = 128 two.
// ROT: a caller-given rotation (the rotated queries come from qrot_kernel);
// W: the compressed tier's code width.
template <int D, bool ROT, int W>
__global__ __launch_bounds__(kCThreads, D == 64 ? 3 : 2) void chunk_split_kernel(AttnParams p, int nrg) {
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
    chunk_split<D, true, ROT, W>(p, smem, b, kv, rg, sx, start, end, el);
  else
    chunk_split<D, false, false, 4>(p, smem, b, kv, rg, sx, start, end, el);
}

// ---- merge: one wave per (sequence, query token, query head).  With a
// given rotation a workgroup takes kRotMergeRows rows and holds R in LDS for
// their R^T step.
constexpr int kRotMergeRows = 16;

template <int D, bool ROT>
__global__ __launch_bounds__(ROT ? 64 * kRotMergeRows : 256) void chunk_merge_kernel(AttnParams p) {
  constexpr int E = D / 64, ROWS = ROT ? kRotMergeRows : 4;
  // R (D x D floats) in dynamic LDS, given at launch with a rotation only
  extern __shared__ __attribute__((aligned(16))) float rsh[];
  if constexpr (ROT) {
    // R staged before any wave can leave, all of a thread's loads in flight together
    constexpr int PER = D * D / 4 / (64 * ROWS);
    static_assert(PER * 64 * ROWS * 4 == D * D, "R staging covers the matrix");
    float4v x[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) x[u] = reinterpret_cast<const float4v*>(p.rot)[threadIdx.x + u * 64 * ROWS];
#pragma unroll
    for (int u = 0; u < PER; ++u) reinterpret_cast<float4v*>(rsh)[threadIdx.x + u * 64 * ROWS] = x[u];
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int rowq = blockIdx.x * ROWS + (threadIdx.x >> 6), b = blockIdx.y;
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
  const size_t firstq = base, firste = base + (size_t)p.Sq * R;
  // Splits are taken kMU at a time, ascending, with every load of a group
  // (and the first group of both tiers) issued before any is used: one
  // memory round trip covers up to kMU splits per tier.  A group's largest
  // log-sum-exp rescales the running sums when it raises their reference; a
  // split with no scores (-inf) or a NaN is selected out, never multiplied
  // by zero.
  constexpr int kMU = 4;
  struct Tier {
    float m = neg_inf(), wsum = 0.0f, acc[E] = {};
    bool nan = false;
  } tr[2];
  // splits past the tier's last are read at a clamped, existing row (every
  // call has at least one split row) and masked, so no load is conditional
  auto load = [&](size_t first, int n, int s0, float (&l)[kMU], float (&x)[kMU][E]) {
#pragma unroll
    for (int u = 0; u < kMU; ++u) {
      const bool in = s0 + u < n;
      const size_t r = first + (size_t)min(s0 + u, max(n - 1, 0)) * R;
      const float lv = p.part_lse[r];
      l[u] = in ? lv : neg_inf();
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float xv = p.part_o[r * D + lane + 64 * e];
        x[u][e] = in ? xv : 0.0f;
      }
    }
  };
  auto fold = [&](Tier& t, const float (&l)[kMU], const float (&x)[kMU][E]) {
    float mc = neg_inf();
#pragma unroll
    for (int u = 0; u < kMU; ++u) {
      t.nan |= l[u] != l[u];
      mc = fmaxf(mc, l[u]);
    }
    if (mc > t.m) {
      const float f = (t.m == neg_inf()) ? 0.0f : __expf(t.m - mc);
      t.wsum *= f;
#pragma unroll
      for (int e = 0; e < E; ++e) t.acc[e] *= f;
      t.m = mc;
    }
    if (t.m == neg_inf()) return;
#pragma unroll
    for (int u = 0; u < kMU; ++u) {
      const bool ok = l[u] > neg_inf();
      const float wt = __expf(l[u] - t.m);
      t.wsum += ok ? wt : 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) t.acc[e] += ok ? wt * x[u][e] : 0.0f;
    }
  };
  {
    float lq[kMU], xq[kMU][E], le[kMU], xe[kMU][E];
    load(firstq, nq, 0, lq, xq);
    load(firste, ne, 0, le, xe);
    fold(tr[0], lq, xq);
    fold(tr[1], le, xe);
    for (int s0 = kMU; s0 < nq; s0 += kMU) {
      load(firstq, nq, s0, lq, xq);
      fold(tr[0], lq, xq);
    }
    for (int s0 = kMU; s0 < ne; s0 += kMU) {
      load(firste, ne, s0, le, xe);
      fold(tr[1], le, xe);
    }
  }
  float res_o[2][E], res_l[2];
#pragma unroll
  for (int tier = 0; tier < 2; ++tier) {
    const Tier& t = tr[tier];
#pragma unroll
    for (int e = 0; e < E; ++e) res_o[tier][e] = (t.m == neg_inf()) ? 0.0f : t.acc[e] / t.wsum;
    res_l[tier] = t.nan ? __builtin_nanf("") : (t.m == neg_inf() ? neg_inf() : t.m + __logf(t.wsum));
  }
  // inverse rotation of the compressed-tier output: dim = lane + 64e
  float rd = inv_sqrt_d(D);
  if constexpr (ROT) {
    // R^T o_rot: dim t of the result is sum_k R[k][t] o_rot[k], in four
    // ascending partial sums (k mod 4) added in order, each o_rot[k] read
    // from the lane that holds it
    float acc[4][E];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[j][e] = 0.0f;
#pragma unroll 4
    for (int k0 = 0; k0 < D; k0 += 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = k0 + j;
        const float ok = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, (k < 64) ? res_o[0][0] : res_o[0][E - 1]), k & 63));
#pragma unroll
        for (int e = 0; e < E; ++e) acc[j][e] = fmaf(rsh[k * D + lane + 64 * e], ok, acc[j][e]);
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) res_o[0][e] = (acc[0][e] + acc[1][e]) + (acc[2][e] + acc[3][e]);
    rd = 1.0f;
  } else {
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
  }
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

hipError_t launch_decode_qrot(const AttnParams& p, int D, hipStream_t stream);

template <int D, bool ROT>
static void launch_chunk_split_w(const AttnParams& p, dim3 grid, int nrg, hipStream_t stream) {
  if (p.qw == 2)
    hipLaunchKernelGGL((chunk_split_kernel<D, ROT, 2>), grid, dim3(kCThreads), 0, stream, p, nrg);
  else if (p.qw == 3)
    hipLaunchKernelGGL((chunk_split_kernel<D, ROT, 3>), grid, dim3(kCThreads), 0, stream, p, nrg);
  else
    hipLaunchKernelGGL((chunk_split_kernel<D, ROT, 4>), grid, dim3(kCThreads), 0, stream, p, nrg);
}
template <int D>
static void launch_chunk_split(const AttnParams& p, dim3 grid, int nrg, hipStream_t stream) {
  if (p.rot)
    launch_chunk_split_w<D, true>(p, grid, nrg, stream);
  else
    launch_chunk_split_w<D, false>(p, grid, nrg, stream);
}

hipError_t launch_chunk(const AttnParams& p, int D, hipStream_t stream) {
  hipError_t qe = launch_decode_qrot(p, D, stream);
  if (qe != hipSuccess) return qe;
  const int R = p.Tq * p.G;
  const int nrg = (R + kRowsPerWG - 1) / kRowsPerWG;
  const dim3 grid(p.Hkv * nrg, p.Sq + p.Se, p.B);
  const dim3 mgrid((p.Tq * p.Hq + 3) / 4, p.B), rgrid((p.Tq * p.Hq + kRotMergeRows - 1) / kRotMergeRows, p.B);
  if (D == 64) {
    launch_chunk_split<64>(p, grid, nrg, stream);
    if (p.rot)
      hipLaunchKernelGGL((chunk_merge_kernel<64, true>), rgrid, dim3(64 * kRotMergeRows), 64 * 64 * sizeof(float),
                         stream, p);
    else
      hipLaunchKernelGGL((chunk_merge_kernel<64, false>), mgrid, dim3(256), 0, stream, p);
  } else {
    launch_chunk_split<128>(p, grid, nrg, stream);
    if (p.rot)
      hipLaunchKernelGGL((chunk_merge_kernel<128, true>), rgrid, dim3(64 * kRotMergeRows), 128 * 128 * sizeof(float),
                         stream, p);
    else
      hipLaunchKernelGGL((chunk_merge_kernel<128, false>), mgrid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace akv
