// Split-KV decode attention over a two-tier history, and the exact
// log-sum-exp merge (ActiveKV, "Context beyond VRAM", "What I built": a
// full-precision recent window and an encoded older tier, attended apart and
// combined without approximation; each partial carries the log-sum-exp statistic that "Bringing a
// serving stack up on new silicon", "What I built", adds to the
// paged-attention path).
//
// One workgroup (4 waves) per (split, kv head, sequence).  A split is a fixed
// run of P tokens of one tier; the waves take its 64-token blocks round-robin.
// The G <= 8 query heads sharing the kv head are the columns of 16x16x32
// matrix-core tiles:
//   scores:  D[token][col] = K_tile[token][dims] x Q[dims][col]
//   values:  O^T[dim][col] += V^T[dim][tokens] x P^T[tokens][col]
// Compressed tier (QuantForge walkthrough, section 1: the query is rotated
// once instead of inverse-rotating blocks): the query is rotated by the
// Walsh-Hadamard butterflies in fp32 (or, for a caller-given rotation R, read
// from a small kernel that forms R q once per call) and split into fp16 hi +
// lo parts held in columns 0..7 and 8..15, so the score keeps ~fp32
// precision.  K codes are expanded through an LDS table into fp16 hi and lo
// parts of the Lloyd-Max levels (two tiles per group) and the fp16 group
// scale multiplies the fp32 group partial score; V codes enter the value tile
// as fp16 levels, their group scale multiplying the probabilities instead.
// The table has one 256-byte row per table field (two codes): 32 copies of
// the (level, level) fp16 hi pair, then 32 copies of the lo pair; lane l
// reads copy l % 32, which keeps the random-row lookups of a wave free of
// bank conflicts.  Code widths 2 and 3 use the same fields (4 or 64 rows'
// worth of the 4- or 8-level table).  One register buffer per wave holds a
// block; the next block's K codes and scales are requested as soon as the
// scores are done and its V codes once the values are; a wave's issue
// priority falls as it finishes blocks, so waves that are behind issue
// first.  The value sum stays in rotated space.  Exact tier: bf16 K and q feed bf16 tiles directly
// (exact products), and the dim-major V layout makes each lane's V^T operand
// one 16-byte load; two 32-token units per wave, one in flight while the
// other is computed.  Each wave keeps an online softmax (base 2); the four
// waves merge in a fixed order.
//
// A second kernel merges each (sequence, query head)'s partials: compressed-
// tier splits (rotated space), one inverse rotation per head (R^T for a
// given rotation), exact-tier splits, then the two tiers.  Its reduction
// tree is fixed, so repeated runs are bit-identical.
#include "akv_common.h"
#include "akv_params.h"

namespace akv {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMainLds = 65536;               // LUT / epilogue scratch
constexpr int kScaleStage = 1056;             // per wave: two units' K and V scales (1024 B used)
constexpr int kLdsBytes = kMainLds + kWaves * kScaleStage;

__device__ inline float4v mfma16(half8 a, half8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ inline float4v mfma16bf(bf16x8 a, bf16x8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Lane exchanges inside rows of 16 lanes through DPP (VALU, no LDS):
// quad_perm [1,0,3,2] / [2,3,0,1] give lane l ^ 1 / l ^ 2; row_ror:r gives
// lane (l - r) mod 16, so l ^ 4 is row_ror:4 on lanes with bit 2 set and
// row_ror:12 on the others, and l ^ 8 is row_ror:8.
template <int CTRL>
__device__ inline float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ inline float xor1(float x) { return dpp_mov<0xB1>(x); }
__device__ inline float xor2(float x) { return dpp_mov<0x4E>(x); }
__device__ inline float xor4(float x) {
  const float a = dpp_mov<0x124>(x), b = dpp_mov<0x12C>(x);
  return (threadIdx.x & 4) ? a : b;
}
__device__ inline float xor8(float x) { return dpp_mov<0x128>(x); }
// value of lane (l ^ 8) within each row of 16 lanes
__device__ inline float row_swap8(float x) { return xor8(x); }

__device__ inline half2v u32_as_h2(uint32_t x) { return __builtin_bit_cast(half2v, x); }
__device__ inline uint32_t h2_as_u32(half2v x) { return __builtin_bit_cast(uint32_t, x); }

// LDS byte address of the level-table row of code byte k of w, plus off:
// (byte k of w) * 256 + off, built with one byte permute.
template <int k>
__device__ inline uint32_t lut_addr(uint32_t w, uint32_t off) {
  return __builtin_amdgcn_perm(w, off, 0x0C0C0000u | ((4u + k) << 8));
}

// Issue priority from progress: a wave that has finished fewer blocks issues
// first.  Two compressed-tier workgroups share each compute unit, and with
// equal priority the older one's waves win every tie, so the younger one
// falls a block behind and ends alone.
__device__ inline void progress_prio(int k) {
  if (k <= 0) __builtin_amdgcn_s_setprio(3);
  else if (k == 1) __builtin_amdgcn_s_setprio(2);
  else if (k == 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

struct SoftmaxState {
  float m;  // running max (log2 units)
  float l;  // this lane's share of the running sum
};

// Value held by lane (l ^ 32) / lane (l ^ 16), through the gfx950 lane-swap
// instructions (VALU, no LDS traffic).
__device__ inline float xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ inline float xor16(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 16) ? r[0] : r[1]);
}

// Value held by lane l ^ h (h a power of two below 64), all on the VALU.
template <int H>
__device__ inline float lane_xor(float x) {
  if constexpr (H == 1) return xor1(x);
  else if constexpr (H == 2) return xor2(x);
  else if constexpr (H == 4) return xor4(x);
  else if constexpr (H == 8) return xor8(x);
  else if constexpr (H == 16) return xor16(x);
  else return xor32(x);
}

// One butterfly stage across lanes: (a, b) -> (a + b, a - b) with a on the
// lane whose bit H is clear.
template <int H>
__device__ inline float lane_butterfly(float x, int lane) {
  const float o = lane_xor<H>(x);
  return (lane & H) ? (o - x) : (x + o);
}

// Online-softmax step on N scores of one head held by this lane; the running
// max is shared by the 4 lanes (rows 0..3 of 16) with the same column.
// Returns the factor the running output must be scaled by.
template <int N>
__device__ inline float softmax_step(SoftmaxState& st, const float (&s)[N], float (&p)[N]) {
  float t[N];
#pragma unroll
  for (int e = 0; e < N; ++e) t[e] = s[e];
#pragma unroll
  for (int h = N / 2; h >= 1; h >>= 1)  // pairwise tree
#pragma unroll
    for (int e = 0; e < h; ++e) t[e] = fmaxf(t[e], t[e + h]);
  float mx = t[0];
  mx = fmaxf(mx, xor16(mx));
  mx = fmaxf(mx, xor32(mx));
  float mnew = fmaxf(st.m, mx);
  float muse = (mnew == neg_inf()) ? 0.0f : mnew;
  float alpha = __builtin_amdgcn_exp2f(st.m - muse);
  float sum = 0.0f;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    p[e] = __builtin_amdgcn_exp2f(s[e] - muse);
    sum += p[e];
  }
  st.l = st.l * alpha + sum;
  st.m = mnew;
  return alpha;
}

// Scale the running output unless no lane's running max moved.
template <int NT>
__device__ inline void rescale(float4v (&O)[NT], float alpha) {
  if (__ballot(alpha != 1.0f)) {
#pragma unroll
    for (int t = 0; t < NT; ++t) O[t] *= alpha;
  }
}

struct Lds {
  unsigned char* main;   // kMainLds bytes
  unsigned char* stage;  // kWaves x kScaleStage scale staging
};

__device__ inline Lds lds_layout(unsigned char* smem) {
  Lds L;
  L.main = smem;
  L.stage = smem + kMainLds;
  return L;
}

// This wave's pool block ids: lane k holds the id of the wave's blocks k and
// k + 64 (the wave takes blocks w, w + 4, ... of the split).
struct WaveBlocks {
  int lo, hi;
  __device__ inline int get(int i) const {
    return i < 64 ? __builtin_amdgcn_readlane(lo, i) : __builtin_amdgcn_readlane(hi, i - 64);
  }
};

// table == nullptr: the identity table (block k of the tier is pool block k).
__device__ inline WaveBlocks load_wave_blocks(const int* table, int blk0, int nblk_w, int w, int lane) {
  WaveBlocks wb;
  const int k0 = blk0 + w + kWaves * lane, k1 = k0 + kWaves * 64;
  wb.lo = lane < nblk_w ? (table ? table[k0] : k0) : -1;
  wb.hi = lane + 64 < nblk_w ? (table ? table[k1] : k1) : -1;
  return wb;
}

// The block ids a wave may take in a split of P tokens starting at block
// blk0, read before the tier length is known: the table row of tmax entries
// bounds the read, so it can be in flight together with the length load.
__device__ inline WaveBlocks load_split_blocks(const int* row, int tmax, int blk0, int P, int w, int lane) {
  const int cap = min(P >> 6, tmax - blk0);
  return load_wave_blocks(row, blk0, cap > w ? (cap - w + kWaves - 1) / kWaves : 0, w, lane);
}

// Keep the ids of the wave's first nblk_w blocks only.
__device__ inline WaveBlocks trim_blocks(WaveBlocks wb, int nblk_w, int lane) {
  wb.lo = lane < nblk_w ? wb.lo : -1;
  wb.hi = lane + 64 < nblk_w ? wb.hi : -1;
  return wb;
}

// Both tier lengths of sequence b; false if either lies outside its table
// (the sequence's splits then write nothing and the merge reports NaN).
__device__ inline bool tier_lengths(const AttnParams& p, int b, int& ql, int& el) {
  ql = p.qlen_fixed >= 0 ? p.qlen_fixed : (p.qmax ? p.qlen[b] : 0);
  el = p.emax ? p.elen[b] : 0;
  return ql >= 0 && ql <= p.qmax * 64 && el >= 0 && el <= p.emax * 64;
}

// Decode partials are laid out per query head: row ((b * Hkv + kv) * G + g)
// * (Sq + Se) + split, so one head's splits are contiguous for the merge.
__device__ inline size_t part_row(const AttnParams& p, int b, int kv, int g, int sx) {
  return ((size_t)(b * p.Hkv + kv) * p.G + g) * p.part_stride + sx;
}

// ------------------------------------------------------------------ epilogue
// Merge the 4 waves' (m, l, O) of this workgroup and write the split partial.
template <int D>
__device__ void split_epilogue(const AttnParams& p, const Lds& L, int b, int kv, int sx, const SoftmaxState& st,
                               const float4v (&O)[D / 16], bool poison) {
  constexpr int NT = D / 16, C4 = D / 4;
  constexpr int OP = D + 4;  // padded rows: the 8 heads' float4 stores of one wave hit distinct banks
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j = lane & 15, qq = lane >> 4;
  float* sm_m = reinterpret_cast<float*>(L.main);          // [4][8]
  float* sm_l = sm_m + kWaves * 8;                          // [4][8]
  int* sm_bad = reinterpret_cast<int*>(sm_l + kWaves * 8);  // [4]
  float* sm_o = reinterpret_cast<float*>(L.main + 512);     // [4][8][OP]
  float l = st.l;
  l += xor16(l);
  l += xor32(l);
  __syncthreads();  // everyone is done with the LUT / staging region
  if (j < 8) {
    // lane (col j, qq) holds O^T[16t + 4qq + r][j]: one float4 of head j per t
#pragma unroll
    for (int t = 0; t < NT; ++t) *reinterpret_cast<float4v*>(sm_o + (w * 8 + j) * OP + 16 * t + 4 * qq) = O[t];
    if (qq == 0) {
      sm_m[w * 8 + j] = st.m;
      sm_l[w * 8 + j] = l;
    }
  }
  if (lane == 0) sm_bad[w] = poison ? 1 : 0;
  __syncthreads();
  const int G = p.G;
  const bool bad = sm_bad[0] | sm_bad[1] | sm_bad[2] | sm_bad[3];
  for (int idx = tid; idx < G * C4; idx += kThreads) {
    const int g = idx / C4, c4 = idx - g * C4;
    float M = neg_inf();
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, sm_m[v * 8 + g]);
    float4v o;
    float lse;
    if (bad) {
      lse = __builtin_nanf("");
      o = float4v{1, 1, 1, 1} * lse;
    } else if (M == neg_inf()) {
      o = float4v{0, 0, 0, 0};
      lse = neg_inf();
    } else {
      float Lsum = 0.0f;
      float4v acc = float4v{0, 0, 0, 0};
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const float wv = __builtin_amdgcn_exp2f(sm_m[v * 8 + g] - M);
        Lsum += wv * sm_l[v * 8 + g];
        acc += wv * *reinterpret_cast<const float4v*>(sm_o + (v * 8 + g) * OP + 4 * c4);
      }
      o = acc * (1.0f / Lsum);
      lse = (M + __builtin_log2f(Lsum)) * kLn2;
    }
    const size_t prow = part_row(p, b, kv, g, sx);
    *reinterpret_cast<float4v*>(p.part_o + prow * D + 4 * c4) = o;
    if (c4 == 0) p.part_lse[prow] = lse;
  }
}

// ------------------------------------------------------------- quant tier
// Code words of one 32-token unit at code width W (layouts in include/akv.h).
// W = 4: one dword per (tile, group) of K and per value tile of V, each byte
// one table field (two codes).  W < 4: dwords of the pair plane, each byte
// the fields of two groups (K) or two value tiles (V) in its nibbles, and
// for W = 3 the high-plane bits, merged into the fields when used.
template <int D, int W>
struct QUnit {
  static constexpr int KW = W == 4 ? D / 32 : D / 64;
  static constexpr int VW = W == 4 ? D / 16 : D / 32;
  uint32_t kw[2][KW];      // K code dwords: [tile][group or group pair]
  uint32_t vw[VW];         // V code dwords: [value tile or tile pair]
  uint32_t kh[2];          // W = 3: K high-plane bits of each tile (d = 64: 16 bits)
  uint32_t vh[D / 64];     // W = 3: V high-plane dwords (4 value tiles each)
  u32x4 sc;                // this lane's 16-byte slice of the unit's K|V scales
};

// Issue the loads of one 32-token unit (half c of pool block pb).
// PARTS: 1 = K codes and (with the first unit) the block's scales, 2 = V
// codes, 3 = both.
template <int D, int W, int PARTS = 3>
__device__ inline void quant_load(QUnit<D, W>& u, const AttnParams& p, int pb, int kv, int c, int j, int qq,
                                  int lane) {
  constexpr int M = D / 32, NT = D / 16;
  const unsigned char* kcs = p.kc + (size_t)pb * p.q_code_stride + (size_t)kv * (8 * W * D);
  const unsigned char* vcs = p.vc + (size_t)pb * p.q_code_stride + (size_t)kv * (8 * W * D);
#pragma unroll
  for (int tp = 0; tp < 2; ++tp) {
    if constexpr (!(PARTS & 1)) break;
    int row = 32 * c + 8 * (j >> 2) + 4 * tp + (j & 3);
    if constexpr (W == 4) {
      const unsigned char* src = kcs + row * (D / 2) + (D / 8) * qq;
      if constexpr (M == 4) {
        u32x4 x = stream_load<u32x4>(src);
        u.kw[tp][0] = x[0]; u.kw[tp][1] = x[1]; u.kw[tp][2] = x[2]; u.kw[tp][3] = x[3];
      } else {
        u32x2 x = stream_load<u32x2>(src);
        u.kw[tp][0] = x[0]; u.kw[tp][1] = x[1];
      }
    } else {
      const unsigned char* src = kcs + row * (D / 4) + (D / 16) * qq;
      if constexpr (M == 4) {
        u32x2 x = stream_load<u32x2>(src);
        u.kw[tp][0] = x[0]; u.kw[tp][1] = x[1];
      } else {
        u.kw[tp][0] = stream_load<uint32_t>(src);
      }
      if constexpr (W == 3) {
        const unsigned char* hsrc = kcs + 16 * D + row * (D / 8) + (D / 32) * qq;
        if constexpr (M == 4)
          u.kh[tp] = stream_load<uint32_t>(hsrc);
        else
          u.kh[tp] = stream_load<uint16_t>(hsrc);
      }
    }
  }
  if constexpr (!(PARTS & 2)) {
  } else if constexpr (W == 4) {
    // tiles 4v .. 4v + 3 of lane l: 16 bytes at 1 KB v + 16 l of the half
    const u32x4* vsrc = reinterpret_cast<const u32x4*>(vcs + c * 16 * D) + lane;
#pragma unroll
    for (int v = 0; v < NT / 4; ++v) {
      u32x4 x = stream_load<u32x4>(vsrc + 64 * v);
      u.vw[4 * v] = x[0]; u.vw[4 * v + 1] = x[1]; u.vw[4 * v + 2] = x[2]; u.vw[4 * v + 3] = x[3];
    }
  } else {
    const unsigned char* vsrc = vcs + ((c * 4 + qq) * 16 + j) * (D / 8);
    if constexpr (NT == 8) {
      u32x4 x = stream_load<u32x4>(vsrc);
      u.vw[0] = x[0]; u.vw[1] = x[1]; u.vw[2] = x[2]; u.vw[3] = x[3];
    } else {
      u32x2 x = stream_load<u32x2>(vsrc);
      u.vw[0] = x[0]; u.vw[1] = x[1];
    }
    if constexpr (W == 3) {
      const unsigned char* hsrc = vcs + 16 * D + ((c * 4 + qq) * 16 + j) * (D / 16);
      if constexpr (NT == 8) {
        u32x2 x = stream_load<u32x2>(hsrc);
        u.vh[0] = x[0]; u.vh[1] = x[1];
      } else {
        u.vh[0] = stream_load<uint32_t>(hsrc);
      }
    }
  }
  // scales of the whole block, with the first unit: M K-groups then M
  // V-groups, 128 bytes (64 tokens) each; lane (seg, part) carries bytes
  // [16 part, 16 part + 16) of segment seg, so the load reads whole lines
  if ((PARTS & 1) && c == 0) {
    const int lm = lane & (16 * M - 1), seg = lm >> 3, g = seg % M;
    const uint16_t* sb = (seg < M ? p.ks : p.vs) + (size_t)pb * p.q_scale_stride + (size_t)kv * (2 * D) + g * 64 +
                         8 * (lane & 7);
    u.sc = stream_load<u32x4>(sb);
  }
}

// Table fields (one per byte, two codes each) of K group m of tile tp and of
// value tile t.  At W = 3 a field is the pair-plane nibble with the two top
// bits above it (bits 4, 5).
template <int D, int W>
__device__ inline uint32_t kfields(const QUnit<D, W>& u, int tp, int m) {
  if constexpr (W == 4) {
    return u.kw[tp][m];
  } else {
    uint32_t f = (u.kw[tp][m >> 1] >> (4 * (m & 1))) & 0x0F0F0F0Fu;
    if constexpr (W == 3) {
      uint32_t h = u.kh[tp];
      if constexpr (D == 64)  // nibble b of the 16 bits -> byte b
        h = (h & 0xFu) | ((h << 4) & 0xF00u) | ((h << 8) & 0xF0000u) | ((h << 12) & 0xF000000u);
      f |= ((h >> (2 * m)) & 0x03030303u) << 4;
    }
    return f;
  }
}
template <int D, int W>
__device__ inline uint32_t vfields(const QUnit<D, W>& u, int t) {
  if constexpr (W == 4) {
    return u.vw[t];
  } else {
    uint32_t f = (u.vw[t >> 1] >> (4 * (t & 1))) & 0x0F0F0F0Fu;
    if constexpr (W == 3) f |= ((u.vh[t >> 2] >> (2 * (t & 3))) & 0x03030303u) << 4;
    return f;
  }
}

// The block's group scales, parked in LDS by the first unit's lanes < 16M
// (2M 128-byte segments: M K-groups, then M V-groups), and read back per
// unit: lane (col, qq) of unit c reads its 8 tokens 32c + 8qq.. of every
// group.
template <int D, int W>
__device__ inline void park_scales(const QUnit<D, W>& u, unsigned char* stage, int lane) {
  constexpr int M = D / 32;
  if (lane < 16 * M) *reinterpret_cast<u32x4*>(stage + 16 * lane) = u.sc;
}
template <int D>
__device__ inline void unit_scales(const unsigned char* stage, int c, int isv, int qq, u32x4 (&sc)[D / 32]) {
  constexpr int M = D / 32;
#pragma unroll
  for (int m = 0; m < M; ++m) sc[m] = *reinterpret_cast<const u32x4*>(stage + 128 * (isv * M + m) + 64 * c + 16 * qq);
}

// Zero the value scales of tokens >= nvalid, so 0 * garbage cannot appear.
template <int D>
__device__ inline void mask_value_scales(u32x4 (&vsc)[D / 32], int nvalid, int qq) {
#pragma unroll
  for (int m = 0; m < D / 32; ++m)
#pragma unroll
    for (int q2 = 0; q2 < 4; ++q2) {
      const int t0 = 8 * qq + 2 * q2;
      uint32_t x = vsc[m][q2];
      if (t0 >= nvalid) x = 0;
      else if (t0 + 1 >= nvalid) x &= 0xFFFFu;
      vsc[m][q2] = x;
    }
}

// Scores (log2 units) of this lane's 8 tokens 8qq + e of one unit.
template <int D, int W>
__device__ inline void quant_scores(const QUnit<D, W>& u, const u32x4 (&ksc)[D / 32], const half8 (&Q)[D / 32],
                                    const unsigned char* lut, uint32_t loff, float (&s)[8]) {
  constexpr int M = D / 32;
#pragma unroll
  for (int tp = 0; tp < 2; ++tp) {
    float acc[4] = {0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint32_t w = kfields<D, W>(u, tp, m);
      const unsigned char* r0 = lut + lut_addr<0>(w, loff);
      const unsigned char* r1 = lut + lut_addr<1>(w, loff);
      const unsigned char* r2 = lut + lut_addr<2>(w, loff);
      const unsigned char* r3 = lut + lut_addr<3>(w, loff);
      half8 khi = __builtin_bit_cast(half8, u32x4{*reinterpret_cast<const uint32_t*>(r0),
                                                  *reinterpret_cast<const uint32_t*>(r1),
                                                  *reinterpret_cast<const uint32_t*>(r2),
                                                  *reinterpret_cast<const uint32_t*>(r3)});
      // keep the hi and lo reads apart: a paired read returns (hi, lo) in
      // adjacent registers, which then need moves into the two operands
      asm volatile("" ::: "memory");
      half8 klo = __builtin_bit_cast(half8, u32x4{*reinterpret_cast<const uint32_t*>(r0 + 128),
                                                  *reinterpret_cast<const uint32_t*>(r1 + 128),
                                                  *reinterpret_cast<const uint32_t*>(r2 + 128),
                                                  *reinterpret_cast<const uint32_t*>(r3 + 128)});
      float4v dm = mfma16(khi, Q[m], float4v{0, 0, 0, 0});
      dm = mfma16(klo, Q[m], dm);
      // group scales of this lane's rows: tokens 8qq + 4tp + r (r = 0..3)
      half2v s01 = u32_as_h2(ksc[m][2 * tp]), s23 = u32_as_h2(ksc[m][2 * tp + 1]);
      acc[0] = fmaf((float)s01[0], dm[0], acc[0]);
      acc[1] = fmaf((float)s01[1], dm[1], acc[1]);
      acc[2] = fmaf((float)s23[0], dm[2], acc[2]);
      acc[3] = fmaf((float)s23[1], dm[3], acc[3]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) s[4 * tp + r] = acc[r];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] += row_swap8(s[e]);  // hi-column + lo-column partial scores
}

// O^T += V'^T P^T for one unit, V'^T[dim][token] = C16[code] * scale.  The
// scale belongs to (token, group), so it multiplies the probabilities
// instead: value tile t (group t / 2) uses P_g = P * scale(., g), and the
// table levels enter the matrix cores as they are (4 multiplies per group
// instead of 4 per tile).
template <int D, int W>
__device__ inline void quant_values(const QUnit<D, W>& u, const u32x4 (&vsc)[D / 32], half8 pb8, const unsigned char* lut,
                                    uint32_t loff, float4v (&O)[D / 16]) {
  constexpr int M = D / 32;
  const u32x4 pw = __builtin_bit_cast(u32x4, pb8);
  half8 pg[M];
#pragma unroll
  for (int g = 0; g < M; ++g) {
    u32x4 x;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = h2_as_u32(u32_as_h2(pw[i]) * u32_as_h2(vsc[g][i]));
    pg[g] = __builtin_bit_cast(half8, x);
  }
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    const uint32_t w = vfields<D, W>(u, t);
    const uint32_t l0 = *reinterpret_cast<const uint32_t*>(lut + lut_addr<0>(w, loff));
    const uint32_t l1 = *reinterpret_cast<const uint32_t*>(lut + lut_addr<1>(w, loff));
    const uint32_t l2 = *reinterpret_cast<const uint32_t*>(lut + lut_addr<2>(w, loff));
    const uint32_t l3 = *reinterpret_cast<const uint32_t*>(lut + lut_addr<3>(w, loff));
    O[t] = mfma16(__builtin_bit_cast(half8, u32x4{l0, l1, l2, l3}), pg[t >> 1], O[t]);
  }
}

// One 64-token block = two 32-token units (a: tokens 0..31, b: 32..63) per
// softmax step: the two units' table reads and matrix-core chains are
// independent, so one wave keeps more of them in flight.  PARTIAL: only
// the first nva / nvb tokens of a / b exist.
// reload_ks() runs once the K codes and the scales are consumed, reload_v()
// once the V codes are: they may request the next block into ua / ub.
template <int D, int W, bool PARTIAL, class RK, class RV>
__device__ inline void quant_block(const QUnit<D, W>& ua, const QUnit<D, W>& ub, int nva, int nvb, const half8 (&Q)[D / 32],
                                   const unsigned char* lut, unsigned char* stage, uint32_t loff, int qq, int lane,
                                   SoftmaxState& st, float4v (&O)[D / 16], RK&& reload_ks, RV&& reload_v) {
  constexpr int M = D / 32;
  // scales of both units (LDS ops of a wave run in order)
  __builtin_amdgcn_wave_barrier();
  u32x4 ksa[M], vsa[M], ksb[M], vsb[M];
  park_scales<D, W>(ua, stage, lane);
  __builtin_amdgcn_wave_barrier();
  unit_scales<D>(stage, 0, 0, qq, ksa);
  unit_scales<D>(stage, 1, 0, qq, ksb);
  float s[16];
  {
    float sa[8], sb[8];
    quant_scores<D, W>(ua, ksa, Q, lut, loff, sa);
    quant_scores<D, W>(ub, ksb, Q, lut, loff, sb);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s[e] = (PARTIAL && 8 * qq + e >= nva) ? neg_inf() : sa[e];
      s[8 + e] = (PARTIAL && 8 * qq + e >= nvb) ? neg_inf() : sb[e];
    }
  }
  reload_ks();
  float pr[16];
  rescale(O, softmax_step<16>(st, s, pr));
  // the value scales only now (fewer registers live through the scores)
  unit_scales<D>(stage, 0, 1, qq, vsa);
  unit_scales<D>(stage, 1, 1, qq, vsb);
  __builtin_amdgcn_wave_barrier();
  if (PARTIAL) {
    mask_value_scales<D>(vsa, nva, qq);
    mask_value_scales<D>(vsb, nvb, qq);
  }
  half8 pa8, pb8;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    pa8[e] = (_Float16)pr[e];
    pb8[e] = (_Float16)pr[8 + e];
  }
  quant_values<D, W>(ua, vsa, pa8, lut, loff, O);
  quant_values<D, W>(ub, vsb, pb8, lut, loff, O);
  reload_v();
}

template <int D, int W>
__device__ void quant_split(const AttnParams& p, const Lds& L, int b, int kv, int sx, int s) {
  constexpr int M = D / 32;   // groups = score tiles per token tile
  constexpr int NT = D / 16;  // value tiles
  constexpr int QV = D / 32;  // query values per lane in the rotation
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j = lane & 15, qq = lane >> 4;
  const int G = p.G;
  unsigned char* smem = L.main;

  // requests first, none waiting for another: this wave's block ids, this
  // lane's query values and the tier lengths
  progress_prio(0);
  const int start = s * p.Pq;
  const int blk0 = start >> 6;
  const WaveBlocks wb_all =
      load_split_blocks(p.qtab ? p.qtab + (size_t)b * p.qmax : nullptr, p.qmax, blk0, p.Pq, w, lane);
  // rotation work split: wave w takes heads 2w, 2w+1; lane holds dims QV*(lane%32).. of head 2w + lane/32
  const int rh = 2 * w + (lane >> 5), rd0 = QV * (lane & 31);
  float qv[QV];
  if (p.rot) {  // rotated once per call by qrot_kernel
    const float* qsrc = p.qrot + ((size_t)b * p.Hq + kv * G + min(rh, G - 1)) * D + rd0;
#pragma unroll
    for (int e = 0; e < QV; ++e) qv[e] = qsrc[e];
  } else {
    const uint16_t* qsrc = p.q + ((size_t)b * p.Hq + kv * G + min(rh, G - 1)) * D + rd0;
#pragma unroll
    for (int e = 0; e < QV; ++e) qv[e] = bf16_bits_to_float(qsrc[e]);
  }
  // the level pair of table field tid (two codes: see kfields), for the
  // level table below
  constexpr int kRows = 1 << (2 * W);
  int i0, i1;
  if constexpr (W == 4) {
    i0 = tid & 15, i1 = tid >> 4;
  } else if constexpr (W == 3) {
    i0 = (tid & 3) | (((tid >> 4) & 1) << 2), i1 = ((tid >> 2) & 3) | (((tid >> 5) & 1) << 2);
  } else {
    i0 = tid & 3, i1 = (tid >> 2) & 3;
  }
  const float c0 = __builtin_bit_cast(float, level_bits<W>()[i0 & ((1 << W) - 1)]);
  const float c1 = __builtin_bit_cast(float, level_bits<W>()[i1 & ((1 << W) - 1)]);
  int ql, el;
  if (!tier_lengths(p, b, ql, el) || start >= ql) return;  // bad lengths, or an idle split
  const int end = min(start + p.Pq, ql);
  const int nblk = ((end + 63) >> 6) - blk0;
  const int nblk_w = (nblk - w + kWaves - 1) / kWaves;
  const WaveBlocks wb = trim_blocks(wb_all, nblk_w, lane);

  // level table (needs nothing loaded): row e (table field) = 256 B: 32 x hi
  // pair | 32 x lo pair; 4^W rows
  if (tid < kRows) {
    const int e = tid;
    _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
    _Float16 l0 = (_Float16)(c0 - (float)h0), l1 = (_Float16)(c1 - (float)h1);
    const uint32_t hip = h2_as_u32(half2v{h0, h1});
    const uint32_t lop = h2_as_u32(half2v{l0, l1});
    uint32_t* row = reinterpret_cast<uint32_t*>(smem) + e * 64;
    const u32x4 h4 = u32x4{hip, hip, hip, hip}, l4 = u32x4{lop, lop, lop, lop};
#pragma unroll
    for (int k = 0; k < 32; k += 4) {
      const int slot = (k + 4 * (e & 7)) & 31;  // 8 consecutive rows' stores start in distinct banks
      *reinterpret_cast<u32x4*>(row + slot) = h4;
      *reinterpret_cast<u32x4*>(row + 32 + slot) = l4;
    }
  }

  // the first block's loads as soon as the block ids are in; the loads are
  // unconditional (a bad id reads block 0 and poisons the split), so the
  // compiler's wait counts stay exact instead of draining all loads in
  // flight where paths join
  const int klast = max(nblk_w - 1, 0);
  auto load_block = [&](QUnit<D, W>& u0, QUnit<D, W>& u1, bool& ok, int k) {
    int pb = wb.get(min(k, klast));
    ok = pb >= 0 && pb < p.qnb;
    pb = ok ? pb : 0;
    quant_load<D, W>(u0, p, pb, kv, 0, j, qq, lane);
    quant_load<D, W>(u1, p, pb, kv, 1, j, qq, lane);
  };
  QUnit<D, W> ra0, ra1;
  bool oka;
  load_block(ra0, ra1, oka, 0);

  // rotated, pre-scaled query q' = H q * (RN(1/sqrt d) * scale * log2 e):
  // butterflies inside the lane for h < QV, across lanes (xor h/QV) above
  // (with a given rotation R, q' = (R q) * scale * log2 e, R q already done)
  if (!p.rot) {
#pragma unroll
    for (int h = 1; h < QV; h <<= 1)
#pragma unroll
      for (int e = 0; e < QV; ++e)
        if (!(e & h)) {
          float a = qv[e], c = qv[e + h];
          qv[e] = a + c;
          qv[e + h] = a - c;
        }
#pragma unroll
    for (int e = 0; e < QV; ++e) {
      qv[e] = lane_butterfly<1>(qv[e], lane);
      qv[e] = lane_butterfly<2>(qv[e], lane);
      qv[e] = lane_butterfly<4>(qv[e], lane);
      qv[e] = lane_butterfly<8>(qv[e], lane);
      qv[e] = lane_butterfly<16>(qv[e], lane);
    }
  }
  const float qmul = (p.rot ? 1.0f : inv_sqrt_d(D)) * p.qscale2;
  // staged q' rows of D + 4 floats: the 8 rows read by one 128-bit LDS read
  // start in distinct banks
  constexpr int QP = D + 4;
  float* qf = reinterpret_cast<float*>(L.stage);  // [8][QP] floats, reuses the scale stage area
  static_assert(kWaves * kScaleStage >= 8 * (128 + 4) * 4, "query staging does not fit");
  if (rh < G) {
    float* dst = qf + rh * QP + rd0;
    if constexpr (QV == 4)
      *reinterpret_cast<float4v*>(dst) = float4v{qv[0] * qmul, qv[1] * qmul, qv[2] * qmul, qv[3] * qmul};
    else
#pragma unroll
      for (int e = 0; e < QV; ++e) dst[e] = qv[e] * qmul;
  }
  __syncthreads();
  half8 Q[M];
  {
    const int hj = j & 7;
    const bool lopart = j >= 8;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float* src = qf + hj * QP + 32 * m + 8 * qq;
      float4v a = *reinterpret_cast<const float4v*>(src);
      float4v c = *reinterpret_cast<const float4v*>(src + 4);
      if (hj >= G) a = c = float4v{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = e < 4 ? a[e] : c[e - 4];
        _Float16 hi = (_Float16)v;
        _Float16 lo = (_Float16)(v - (float)hi);
        Q[m][e] = lopart ? lo : hi;
      }
    }
  }
  __syncthreads();  // the query area becomes the scale stage
  const uint32_t loff = 4 * (lane & 31);  // this lane's table copy

  SoftmaxState st{neg_inf(), 0.0f};
  float4v O[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) O[t] = float4v{0, 0, 0, 0};
  bool poison = false;
  unsigned char* stage = L.stage + w * kScaleStage;
  // block k of this wave covers tokens tb .. tb + 63; a bad block id poisons
  // the split (its partial becomes NaN), the loads then read block 0
  // one register buffer per wave, refilled in two parts while its block is
  // computed: the next block's K codes and scales once the scores are done,
  // its V codes once the values are (a second whole buffer measured slower:
  // it pushes the kernel to 256 VGPRs and spills).  Only a wave's last block
  // (which may be the split's partial one) requests nothing.
  for (int k = 0; k + 1 < nblk_w; ++k) {
    progress_prio(k);
    poison |= !oka;
    int pbn = wb.get(k + 1);
    const bool okn = pbn >= 0 && pbn < p.qnb;
    pbn = okn ? pbn : 0;
    auto rks = [&]() {
      quant_load<D, W, 1>(ra0, p, pbn, kv, 0, j, qq, lane);
      quant_load<D, W, 1>(ra1, p, pbn, kv, 1, j, qq, lane);
    };
    auto rv = [&]() {
      quant_load<D, W, 2>(ra0, p, pbn, kv, 0, j, qq, lane);
      quant_load<D, W, 2>(ra1, p, pbn, kv, 1, j, qq, lane);
    };
    quant_block<D, W, false>(ra0, ra1, 32, 32, Q, smem, stage, loff, qq, lane, st, O, rks, rv);
    oka = okn;
  }
  if (nblk_w > 0) {
    progress_prio(nblk_w - 1);
    const int tb = (blk0 + w + kWaves * (nblk_w - 1)) * 64;
    poison |= !oka;
    auto none = []() {};
    if (end - tb >= 64)
      quant_block<D, W, false>(ra0, ra1, 32, 32, Q, smem, stage, loff, qq, lane, st, O, none, none);
    else
      quant_block<D, W, true>(ra0, ra1, min(end - tb, 32), max(end - tb - 32, 0), Q, smem, stage, loff, qq, lane,
                              st, O, none, none);
  }
  split_epilogue<D>(p, L, b, kv, sx, st, O, poison);
}

// ------------------------------------------------------------- exact tier
template <int D>
struct EUnit {
  u32x4 kx[2][D / 32];  // K rows of both 16-token tiles
  u32x4 vx[D / 16];     // V^T operand of value tile t: 8 tokens of dim 16t + j
};

// Issue the loads of one 32-token unit (half c of pool block pb).  K is
// token-major: score tile m takes dims 8 (4m + qq) .. + 7 on lane (row j,
// qq), so one load instruction reads 64 consecutive bytes of each of its 16
// rows (the query operand uses the same dim order).  V is dim-major inside
// each half block, so the same lane reads tokens 32c + 8qq .. + 7 of dim
// 16t + j, 1 KB of consecutive bytes per load instruction.  Both operands
// come straight from HBM, with no transposition.  NTV: the V loads are
// non-temporal (each V load instruction reads 1 KB of whole lines; K rows are
// read in 64-byte pieces by four instructions, so they keep normal loads).
template <int D, bool NTV>
__device__ inline void exact_load(EUnit<D>& u, const AttnParams& p, int pb, int kv, int c, int j, int qq, int lane) {
  constexpr int MK = D / 32;
  const uint16_t* kslab = p.ek + ((size_t)pb * p.Hkv + kv) * kBlock * D;
  const uint16_t* vslab = p.ev + ((size_t)pb * p.Hkv + kv) * kBlock * D;
#pragma unroll
  for (int tp = 0; tp < 2; ++tp) {
    int row = 32 * c + 8 * (j >> 2) + 4 * tp + (j & 3);
    const u32x4* src = reinterpret_cast<const u32x4*>(kslab + row * D + 8 * qq);
#pragma unroll
    for (int m = 0; m < MK; ++m) u.kx[tp][m] = src[4 * m];
  }
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    const void* src = vslab + (c * D + 16 * t + j) * (kBlock / 2) + 8 * qq;
    u.vx[t] = NTV ? stream_load<u32x4>(src) : *reinterpret_cast<const u32x4*>(src);
  }
}

template <int D, bool PARTIAL>
__device__ inline void exact_compute(const EUnit<D>& u, int nvalid, const bf16x8 (&Q)[D / 32], float qscale2,
                                     int qq, SoftmaxState& st, float4v (&O)[D / 16]) {
  constexpr int MK = D / 32, NT = D / 16;
  // ---- scores
  float s[8];
#pragma unroll
  for (int tp = 0; tp < 2; ++tp) {
    float4v dm = float4v{0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < MK; ++m) dm = mfma16bf(__builtin_bit_cast(bf16x8, u.kx[tp][m]), Q[m], dm);
#pragma unroll
    for (int r = 0; r < 4; ++r) s[4 * tp + r] = dm[r] * qscale2;
  }
  // missing tokens: score -inf and value 0 (the pool past the length may hold
  // anything, and 0 * NaN would not vanish)
  uint32_t vmask[4] = {~0u, ~0u, ~0u, ~0u};
  if (PARTIAL) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (8 * qq + e >= nvalid) s[e] = neg_inf();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t0 = 8 * qq + 2 * i;
      vmask[i] = t0 >= nvalid ? 0u : (t0 + 1 >= nvalid ? 0xFFFFu : ~0u);
    }
  }
  float pr[8];
  rescale(O, softmax_step(st, s, pr));
  bf16x8 pb8;
#pragma unroll
  for (int e = 0; e < 8; ++e) pb8[e] = (__bf16)pr[e];
  // ---- values: O^T[dim 16t + j] += V^T[dim][tokens 8qq..] x P^T
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    u32x4 x = u.vx[t];
    if (PARTIAL) x = u32x4{x[0] & vmask[0], x[1] & vmask[1], x[2] & vmask[2], x[3] & vmask[3]};
    O[t] = mfma16bf(__builtin_bit_cast(bf16x8, x), pb8, O[t]);
  }
}

template <int D, bool NTV>
__device__ void exact_split(const AttnParams& p, const Lds& L, int b, int kv, int sx, int s) {
  constexpr int MK = D / 32;  // score tiles per token tile
  constexpr int NT = D / 16;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j = lane & 15, qq = lane >> 4;
  const int G = p.G;

  // requests first, as in the compressed tier: block ids, query, lengths
  const int start = s * p.Pe;
  const int blk0 = start >> 6;
  const WaveBlocks wb_all = load_split_blocks(p.etab + (size_t)b * p.emax, p.emax, blk0, p.Pe, w, lane);
  // query operand: lane (col j, qq) holds dims 8 (4m + qq) + e of head j
  bf16x8 Q[MK];
  {
    const int hj = min(j, G - 1);  // padded columns read a valid head, then zero
    const uint16_t* qsrc = p.q + ((size_t)b * p.Hq + kv * G + hj) * D + 8 * qq;
#pragma unroll
    for (int m = 0; m < MK; ++m) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qsrc + 32 * m);
      if (j >= G) x = u32x4{0, 0, 0, 0};
      Q[m] = __builtin_bit_cast(bf16x8, x);
    }
  }
  int ql, el;
  if (!tier_lengths(p, b, ql, el) || start >= el) return;  // bad lengths, or an idle split
  const int end = min(start + p.Pe, el);

  SoftmaxState st{neg_inf(), 0.0f};
  float4v O[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) O[t] = float4v{0, 0, 0, 0};
  bool poison = false;

  const int nblk = ((end + 63) >> 6) - blk0;
  const int nblk_w = (nblk - w + kWaves - 1) / kWaves;
  const WaveBlocks wb = trim_blocks(wb_all, nblk_w, lane);
  // every step loads, past the wave's last block too (that block again), so
  // the wait counts stay exact; a bad block id poisons the split (its
  // partial becomes NaN) and the loads then read block 0
  const int ilast = max(nblk_w - 1, 0);
  auto block_of = [&](int i, bool& ok) {
    int pb = wb.get(min(i, ilast));
    ok = pb >= 0 && pb < p.enb;
    return ok ? pb : 0;
  };
  EUnit<D> ua, ub;
  bool oka, okb;
  exact_load<D, NTV>(ua, p, block_of(0, oka), kv, 0, j, qq, lane);
  for (int i = 0; i < nblk_w; ++i) {
    const int pb = block_of(i, okb);
    exact_load<D, NTV>(ub, p, pb, kv, 1, j, qq, lane);
    const int tb = (blk0 + w + kWaves * i) * 64;
    poison |= !oka;
    if (end - tb >= 32) exact_compute<D, false>(ua, 32, Q, p.qscale2, qq, st, O);
    else exact_compute<D, true>(ua, end - tb, Q, p.qscale2, qq, st, O);
    exact_load<D, NTV>(ua, p, block_of(i + 1, oka), kv, 0, j, qq, lane);
    if (end - tb >= 64) exact_compute<D, false>(ub, 32, Q, p.qscale2, qq, st, O);
    else if (end - tb > 32) exact_compute<D, true>(ub, end - tb - 32, Q, p.qscale2, qq, st, O);
  }
  split_epilogue<D>(p, L, b, kv, sx, st, O, poison);
}

// --------------------------------------------------------------- merging
__device__ inline void merge_two(float oa, float la, float ob, float lb, float& o, float& lse) {
  if (la != la || lb != lb) {
    o = lse = __builtin_nanf("");
    return;
  }
  float M = fmaxf(la, lb);
  if (M == neg_inf()) {
    o = 0.0f;
    lse = neg_inf();
    return;
  }
  float wa = __expf(la - M), wb = __expf(lb - M);
  float W = wa + wb;
  const float rW = 1.0f / W;
  o = (wa * rW) * oa + (wb * rW) * ob;
  lse = M + __logf(W);
}

// The split a workgroup takes (see split_rotate).
__device__ inline int split_of_workgroup(const AttnParams& p) {
  if (!p.split_rotate) return blockIdx.x;
  const int S = p.Sq + p.Se, unit = blockIdx.y + p.Hkv * blockIdx.z;
  return ((int)blockIdx.x + S - unit % S) % S;
}

template <int D, int W>
__global__ __launch_bounds__(kThreads, 2) void split_decode_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];
  const Lds L = lds_layout(smem);
  const int sx = split_of_workgroup(p), kv = blockIdx.y, b = p.b0 + blockIdx.z;
  // the split reads its tier's length itself, in the same round trip as its
  // block ids and query
  if (sx < p.Sq)
    quant_split<D, W>(p, L, b, kv, p.part_base + sx, sx);
  else
    exact_split<D, false>(p, L, b, kv, p.part_base + sx, sx - p.Sq);
}

// A call without a compressed tier: exact-tier splits only, with
// non-temporal V loads (a kernel of its own, so the two-tier kernel's code
// and registers stay as they are).
template <int D>
__global__ __launch_bounds__(kThreads, 2) void exact_decode_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];
  const Lds L = lds_layout(smem);
  const int sx = split_of_workgroup(p), kv = blockIdx.y, b = p.b0 + blockIdx.z;
  exact_split<D, true>(p, L, b, kv, p.part_base + sx, sx - p.Sq);
}

constexpr int kMergeThreads = 512;

// Sum / max over the 64 lanes of a wave in a fixed butterfly order (every
// lane ends with the same value).
__device__ inline float wave_sum(float x) {
  x += xor1(x);
  x += xor2(x);
  x += xor4(x);
  x += xor8(x);
  x += xor16(x);
  x += xor32(x);
  return x;
}
__device__ inline float wave_max(float x) {
  x = fmaxf(x, xor1(x));
  x = fmaxf(x, xor2(x));
  x = fmaxf(x, xor4(x));
  x = fmaxf(x, xor8(x));
  x = fmaxf(x, xor16(x));
  x = fmaxf(x, xor32(x));
  return x;
}

// One workgroup per (query head, sequence):
//   (1) every split's lse goes to LDS while the partial outputs are requested;
//   (2) wave 0 (compressed tier) and wave 1 (exact tier) turn the lse values
//       into weights w_s = exp(lse_s - M) / W, lse = M + ln W (fixed order);
//   (3) thread (phase, float4 column) sums w_s o_s over splits phase,
//       phase + PH, ... with plain FMAs, the phases are added in order;
//   (4) wave 0 inverse-rotates the compressed-tier output (once per head) and
//       merges the two tiers.  With a given rotation R the inverse R^T o is
//       a product of all threads between (3) and (4): thread (slice, float4
//       column) takes rows slice*RR.. of R, requested at the start.
// Inactive splits (past a sequence's length) are skipped, never multiplied,
// so whatever their workspace rows hold cannot leak in.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(AttnParams p) {
  constexpr int C4 = D / 4, PH = kMergeThreads / C4, E = D / 64, K = 8, RR = D / PH;
  __shared__ float wsh[AKV_MAX_SPLITS];
  __shared__ float rot_in[D];  // compressed-tier output in rotated space (given rotation)
  __shared__ float stats[2][3];  // per tier: lse, nan flag, empty flag
  __shared__ __attribute__((aligned(16))) float4v phase[2][PH * C4];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = p.G, kv = h / G, g = h - kv * G;
  const int Sq = p.Sq, S = p.Sq + p.Se;
  float* out = p.o + ((size_t)b * p.Hq + h) * D;
  float* lout = p.lse + (size_t)b * p.Hq + h;
  const size_t base = part_row(p, b, kv, g, 0);
  const int c4 = tid % C4, ph = tid / C4;
  const int ql = p.qmax ? p.qlen[b] : 0;
  const int el = p.emax ? p.elen[b] : 0;
  const bool bad = ql < 0 || ql > 64 * p.qmax || el < 0 || el > 64 * p.emax;
  const int nq = bad ? 0 : (ql + p.Pq - 1) / p.Pq, ne = bad ? 0 : (el + p.Pe - 1) / p.Pe;
  // (1)
  for (int s = tid; s < S; s += kMergeThreads) wsh[s] = p.part_lse[base + s];
  float4v xo[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int s = ph + k * PH;
    xo[k] = *reinterpret_cast<const float4v*>(p.part_o + (base + (s < S ? s : 0)) * D + 4 * c4);
  }
  float4v rr[RR];  // rows ph*RR.. of a given rotation, columns 4*c4..
  if (p.rot) {
#pragma unroll
    for (int r = 0; r < RR; ++r)
      rr[r] = *reinterpret_cast<const float4v*>(p.rot + (size_t)(ph * RR + r) * D + 4 * c4);
  }
  __syncthreads();
  // (2)
  if (w < 2) {
    const int s0 = w ? Sq : 0, n = w ? ne : nq;
    float m = neg_inf(), nan = 0.0f, sum = 0.0f;
    if (n <= 128) {
      // up to two splits per lane, held in registers between the passes
      // (the same operations in the same order as the general loops below)
      const float l0 = lane < n ? wsh[s0 + lane] : neg_inf();
      const float l1 = lane + 64 < n ? wsh[s0 + lane + 64] : neg_inf();
      if (lane < n) {
        if (l0 != l0) nan = 1.0f;
        else m = fmaxf(m, l0);
      }
      if (lane + 64 < n) {
        if (l1 != l1) nan = 1.0f;
        else m = fmaxf(m, l1);
      }
      m = wave_max(m);
      nan = wave_max(nan);
      const float e0 = (m == neg_inf() || l0 != l0) ? 0.0f : __expf(l0 - m);
      const float e1 = (m == neg_inf() || l1 != l1) ? 0.0f : __expf(l1 - m);
      if (lane < n) sum += e0;
      if (lane + 64 < n) sum += e1;
      sum = wave_sum(sum);
      const float r = sum > 0.0f ? 1.0f / sum : 0.0f;
      if (lane < n) wsh[s0 + lane] = e0 * r;
      if (lane + 64 < n) wsh[s0 + lane + 64] = e1 * r;
    } else {
      for (int i = lane; i < n; i += 64) {
        const float l = wsh[s0 + i];
        if (l != l) nan = 1.0f;
        else m = fmaxf(m, l);
      }
      m = wave_max(m);
      nan = wave_max(nan);
      for (int i = lane; i < n; i += 64) {
        const float l = wsh[s0 + i];
        const float e = (m == neg_inf() || l != l) ? 0.0f : __expf(l - m);
        wsh[s0 + i] = e;
        sum += e;
      }
      sum = wave_sum(sum);
      const float r = sum > 0.0f ? 1.0f / sum : 0.0f;
      for (int i = lane; i < n; i += 64) wsh[s0 + i] *= r;
    }
    if (lane == 0) {
      stats[w][0] = (m == neg_inf()) ? neg_inf() : m + __logf(sum);
      stats[w][1] = (bad || nan != 0.0f) ? 1.0f : 0.0f;
    }
  }
  __syncthreads();
  // (3)
  float4v aq = float4v{0, 0, 0, 0}, ae = float4v{0, 0, 0, 0};
  for (int s0 = 0; s0 < S; s0 += K * PH) {
    if (s0) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int s = s0 + ph + k * PH;
        xo[k] = *reinterpret_cast<const float4v*>(p.part_o + (base + (s < S ? s : 0)) * D + 4 * c4);
      }
    }
    // every weight read first (a clamped, existing slot for splits past S),
    // then the sums in the same order with selects instead of branches
    float wv[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int s = s0 + ph + k * PH;
      wv[k] = wsh[s < S ? s : 0];
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int s = s0 + ph + k * PH;
      const bool inq = s < nq, ine = !inq && s >= Sq && s - Sq < ne;
      const float4v t = wv[k] * xo[k];
      aq = inq ? aq + t : aq;
      ae = ine ? ae + t : ae;
    }
  }
  phase[0][ph * C4 + c4] = aq;
  phase[1][ph * C4 + c4] = ae;
  __syncthreads();
  if (p.rot) {
    // R^T o_rot: the phases of o_rot added in order, then per slice
    // sum_k R[k][t] o_rot[k] over its rows in ascending k; the slices'
    // partials replace phase[0], so (4) adds them like phases
    if (tid < D) {
      const float* f0 = reinterpret_cast<const float*>(phase[0]);
      float v = 0.0f;
#pragma unroll
      for (int k = 0; k < PH; ++k) v += f0[k * D + tid];
      rot_in[tid] = v;
    }
    __syncthreads();
    float4v acc = float4v{0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < RR; ++r) acc += rr[r] * rot_in[ph * RR + r];
    phase[0][ph * C4 + c4] = acc;
    __syncthreads();
  }
  if (tid >= 64) return;
  // (4) wave 0: lane l owns dims l + 64 e
  const float* fq = reinterpret_cast<const float*>(phase[0]);
  const float* fe = reinterpret_cast<const float*>(phase[1]);
  float oq[E], oe[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int t = tid + 64 * e;
    float vq = 0.0f, ve = 0.0f;
#pragma unroll
    for (int k = 0; k < PH; ++k) {
      vq += fq[k * D + t];
      ve += fe[k * D + t];
    }
    oq[e] = vq;
    oe[e] = ve;
  }
  // inverse rotation of the compressed-tier output: (H o_rot) * RN(1/sqrt d)
  // (a given rotation's R^T o_rot is already in oq)
  float rd = inv_sqrt_d(D);
  if (p.rot) {
    rd = 1.0f;
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      oq[e] = lane_butterfly<1>(oq[e], tid);
      oq[e] = lane_butterfly<2>(oq[e], tid);
      oq[e] = lane_butterfly<4>(oq[e], tid);
      oq[e] = lane_butterfly<8>(oq[e], tid);
      oq[e] = lane_butterfly<16>(oq[e], tid);
      oq[e] = lane_butterfly<32>(oq[e], tid);
    }
    if (E == 2) {
      float a = oq[0], c = oq[E - 1];
      oq[0] = a + c;
      oq[E - 1] = a - c;
    }
  }
  const bool nanq = stats[0][1] != 0.0f, nane = stats[1][1] != 0.0f;
  const float lq = nanq ? __builtin_nanf("") : stats[0][0];
  const float le = nane ? __builtin_nanf("") : stats[1][0];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float o, lse;
    merge_two(oq[e] * rd, lq, oe[e], le, o, lse);
    out[tid + 64 * e] = o;
    if (tid == 0 && e == 0) *lout = lse;
  }
}

// The merge for calls with at most 128 splits per sequence and the Walsh-
// Hadamard rotation: one workgroup of 4 waves per (query head, sequence),
// one barrier.  Every wave reads all the splits' lse values (lane l: splits
// l and l + 64) and forms both tiers' weights w_s = exp(lse_s - M) / W
// itself, with the same operations in the same order in every wave, so no
// wave waits for another before its weighted sums; wave v sums w_s o_s over
// splits v, v + 4, ... in ascending order, lane l holding dims E l ..
// E l + E - 1 of every split row (one coalesced row per load), each split's
// weight broadcast from the lane that holds it.  Wave 0 then adds the four
// waves' sums in wave order, inverse-rotates the compressed-tier output
// (once per head) and merges the two tiers.  KS = splits per wave (the call's
// split count rounded up); rows past the last split are read at row 0 and
// never used, and inactive splits are skipped, never multiplied.
constexpr int kFastMergeWaves = 4;
constexpr int kFastMergeSplits = 128;

template <int D, int KS>
__global__ __launch_bounds__(64 * kFastMergeWaves) void merge_fast_kernel(AttnParams p) {
  constexpr int E = D / 64;
  static_assert(KS * kFastMergeWaves <= kFastMergeSplits, "lse values are held two per lane");
  __shared__ __attribute__((aligned(16))) float part[kFastMergeWaves][2][D];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G, kv = h / G, g = h - kv * G;
  const int Sq = p.Sq, S = p.Sq + p.Se;
  const size_t base = part_row(p, b, kv, g, 0);
  // every request first: lengths, all lse values, this wave's split rows
  const int ql = p.qmax ? p.qlen[b] : 0;
  const int el = p.emax ? p.elen[b] : 0;
  const float l0 = p.part_lse[base + (lane < S ? lane : 0)];
  const float l1 = p.part_lse[base + (lane + 64 < S ? lane + 64 : 0)];
  float xo[KS][E];
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const int s = w + kFastMergeWaves * k;
    const float* src = p.part_o + (base + (s < S ? s : 0)) * D + E * lane;
    if constexpr (E == 2) {
      const float2 v = *reinterpret_cast<const float2*>(src);
      xo[k][0] = v.x;
      xo[k][1] = v.y;
    } else {
      xo[k][0] = *src;
    }
  }
  const bool bad = ql < 0 || ql > 64 * p.qmax || el < 0 || el > 64 * p.emax;
  const int nq = __builtin_amdgcn_readfirstlane(bad ? 0 : (ql + p.Pq - 1) / p.Pq);
  const int ne = __builtin_amdgcn_readfirstlane(bad ? 0 : (el + p.Pe - 1) / p.Pe);
  // tier weights, in every wave
  const bool q0 = lane < nq, q1 = lane + 64 < nq;
  const bool e0 = lane >= Sq && lane - Sq < ne, e1 = lane + 64 >= Sq && lane + 64 - Sq < ne;
  const bool f0 = l0 == l0, f1 = l1 == l1;
  const bool nanq = __ballot((q0 && !f0) || (q1 && !f1)) != 0;
  const bool nane = __ballot((e0 && !f0) || (e1 && !f1)) != 0;
  float mq = fmaxf((q0 && f0) ? l0 : neg_inf(), (q1 && f1) ? l1 : neg_inf());
  float me = fmaxf((e0 && f0) ? l0 : neg_inf(), (e1 && f1) ? l1 : neg_inf());
  mq = wave_max(mq);
  me = wave_max(me);
  const float x0 = (q0 && f0 && mq != neg_inf()) ? __expf(l0 - mq) : 0.0f;
  const float x1 = (q1 && f1 && mq != neg_inf()) ? __expf(l1 - mq) : 0.0f;
  const float y0 = (e0 && f0 && me != neg_inf()) ? __expf(l0 - me) : 0.0f;
  const float y1 = (e1 && f1 && me != neg_inf()) ? __expf(l1 - me) : 0.0f;
  const float Wq = wave_sum(x0 + x1), We = wave_sum(y0 + y1);
  const float rq = Wq > 0.0f ? 1.0f / Wq : 0.0f, re = We > 0.0f ? 1.0f / We : 0.0f;
  // each split's weight in its own tier (0 for inactive splits, never used)
  const float wt0 = q0 ? x0 * rq : y0 * re;
  const float wt1 = q1 ? x1 * rq : y1 * re;
  float aq[E], ae[E];
#pragma unroll
  for (int e = 0; e < E; ++e) aq[e] = ae[e] = 0.0f;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const int s = w + kFastMergeWaves * k;  // wave-uniform; s < 64 exactly when k < 16
    const float ws = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, k < 64 / kFastMergeWaves ? wt0 : wt1), s & 63));
    if (s < nq) {
#pragma unroll
      for (int e = 0; e < E; ++e) aq[e] = fmaf(ws, xo[k][e], aq[e]);
    } else if (s >= Sq && s - Sq < ne) {
#pragma unroll
      for (int e = 0; e < E; ++e) ae[e] = fmaf(ws, xo[k][e], ae[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    part[w][0][E * lane + e] = aq[e];
    part[w][1][E * lane + e] = ae[e];
  }
  __syncthreads();
  if (w != 0) return;
  float oq[E], oe[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float vq = part[0][0][E * lane + e], ve = part[0][1][E * lane + e];
#pragma unroll
    for (int v = 1; v < kFastMergeWaves; ++v) {
      vq += part[v][0][E * lane + e];
      ve += part[v][1][E * lane + e];
    }
    oq[e] = vq;
    oe[e] = ve;
  }
  // inverse rotation (H o_rot) * RN(1/sqrt d): dim E l + e, bit 0 in the
  // lane when E = 2, the other bits across lanes
  if constexpr (E == 2) {
    const float a = oq[0], c = oq[1];
    oq[0] = a + c;
    oq[1] = a - c;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    oq[e] = lane_butterfly<1>(oq[e], lane);
    oq[e] = lane_butterfly<2>(oq[e], lane);
    oq[e] = lane_butterfly<4>(oq[e], lane);
    oq[e] = lane_butterfly<8>(oq[e], lane);
    oq[e] = lane_butterfly<16>(oq[e], lane);
    oq[e] = lane_butterfly<32>(oq[e], lane);
  }
  const float rd = inv_sqrt_d(D);
  const float lq = (bad || nanq) ? __builtin_nanf("") : (mq == neg_inf() ? neg_inf() : mq + __logf(Wq));
  const float le = (bad || nane) ? __builtin_nanf("") : (me == neg_inf() ? neg_inf() : me + __logf(We));
  float* out = p.o + ((size_t)b * p.Hq + h) * D + E * lane;
  float o[E], lse = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) merge_two(oq[e] * rd, lq, oe[e], le, o[e], lse);
  if constexpr (E == 2)
    *reinterpret_cast<float2*>(out) = float2{o[0], o[1]};
  else
    out[0] = o[0];
  if (lane == 0) p.lse[(size_t)b * p.Hq + h] = lse;
}

// The merge of a decode call: the 4-wave merge where it applies, else the
// general one (more than 128 splits, or a caller-given rotation).
template <int D>
void launch_merge_d(const AttnParams& p, hipStream_t stream) {
  const dim3 mgrid(p.Hq, p.B), fthreads(64 * kFastMergeWaves);
  const int S = p.Sq + p.Se;
  if (p.rot || S > kFastMergeSplits)
    hipLaunchKernelGGL(merge_kernel<D>, mgrid, dim3(kMergeThreads), 0, stream, p);
  else if (S <= 4 * kFastMergeWaves)
    hipLaunchKernelGGL((merge_fast_kernel<D, 4>), mgrid, fthreads, 0, stream, p);
  else if (S <= 8 * kFastMergeWaves)
    hipLaunchKernelGGL((merge_fast_kernel<D, 8>), mgrid, fthreads, 0, stream, p);
  else if (S <= 16 * kFastMergeWaves)
    hipLaunchKernelGGL((merge_fast_kernel<D, 16>), mgrid, fthreads, 0, stream, p);
  else
    hipLaunchKernelGGL((merge_fast_kernel<D, 32>), mgrid, fthreads, 0, stream, p);
}

// --------------------------------------------------------------- standalone merge
// Ascending-order merge of n partials of one row (akv_lse_merge).
__device__ inline void merge_run(const float* po, const float* pl, size_t first, size_t stride, int n, int D,
                                 int t, float& o, float& lse) {
  float M = neg_inf();
  bool nan = false;
  for (int s = 0; s < n; ++s) {
    float x = pl[first + s * stride];
    nan |= (x != x);
    M = fmaxf(M, x);
  }
  if (nan) {
    o = lse = __builtin_nanf("");
    return;
  }
  if (M == neg_inf()) {
    o = 0.0f;
    lse = neg_inf();
    return;
  }
  float W = 0.0f;
  for (int s = 0; s < n; ++s) W += __expf(pl[first + s * stride] - M);
  float acc = 0.0f;
  for (int s = 0; s < n; ++s) {
    size_t r = first + s * stride;
    acc += (__expf(pl[r] - M) / W) * po[r * D + t];
  }
  o = acc;
  lse = M + __logf(W);
}

__global__ __launch_bounds__(256) void lse_merge_kernel(const float* op, const float* lp, int P, int R, int d,
                                                        float* o, float* lse) {
  const int r = blockIdx.x;
  for (int t = threadIdx.x; t < d; t += blockDim.x) {
    float ov, lv;
    merge_run(op, lp, (size_t)r, (size_t)R, P, d, t, ov, lv);
    o[(size_t)r * d + t] = ov;
    if (t == 0) lse[r] = lv;
  }
}

// q' = R q for every (sequence, query token, query head), once per call, when
// the compressed tier uses a given rotation R.  A workgroup takes up to
// kQrotTokens query tokens of one head: their query values are requested
// first; R is staged in LDS (coalesced, rows padded to D + 1 floats so that
// thread i reading row i hits bank (i + k) mod 64) and thread i keeps row i
// in registers; the queries then replace R in LDS and thread i forms
// output i of each, two queries at a time with four partial sums each
// (k mod 4, ascending k, added in order).  NT: tokens per workgroup
// (kQrotTokens for a chunk; 1 for decode, where each of the few workgroups
// reads its rows of R directly).
constexpr int kQrotTokens = 32;

template <int D, int NT>
__global__ __launch_bounds__(D) void qrot_kernel(AttnParams p) {
  __shared__ float rs[NT == 1 ? D : D * (D + 1)];
  static_assert(NT == 1 || NT * D <= D * (D + 1), "the queries fit where R was staged");
  // tokens y NT .. of sequence z, head x: rows (z Tq + t) Hq + x of q and qrot
  const int h = blockIdx.x, i = threadIdx.x;
  const int t0 = blockIdx.y * NT, nt = min(NT, p.Tq - t0);
  const size_t b0 = (size_t)blockIdx.z * p.Tq + t0;
  if constexpr (NT == 1) {
    // one query: thread i reads row i of R straight into registers, the
    // query value requested first so that one round trip covers both
    float* qs = rs;
    const uint16_t q1 = p.q[(b0 * p.Hq + h) * D + i];
    const float4v* row = reinterpret_cast<const float4v*>(p.rot + (size_t)i * D);
    float4v r[D / 4];
#pragma unroll
    for (int k4 = 0; k4 < D / 4; ++k4) r[k4] = row[k4];
    qs[i] = bf16_bits_to_float(q1);
    __syncthreads();
    float acc = 0.0f;
#pragma unroll
    for (int k4 = 0; k4 < D / 4; ++k4)
      acc += r[k4][0] * qs[4 * k4] + r[k4][1] * qs[4 * k4 + 1] + r[k4][2] * qs[4 * k4 + 2] + r[k4][3] * qs[4 * k4 + 3];
    p.qrot[(b0 * p.Hq + h) * D + i] = acc;
  } else {
    uint16_t qb[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) qb[t] = p.q[((b0 + min(t, nt - 1)) * p.Hq + h) * D + i];
#pragma unroll 4
    for (int e = i; e < D * D; e += D) rs[(e / D) * (D + 1) + e % D] = p.rot[e];
    __syncthreads();
    float4v r[D / 4];
#pragma unroll
    for (int k4 = 0; k4 < D / 4; ++k4)
      r[k4] = float4v{rs[i * (D + 1) + 4 * k4], rs[i * (D + 1) + 4 * k4 + 1], rs[i * (D + 1) + 4 * k4 + 2],
                      rs[i * (D + 1) + 4 * k4 + 3]};
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) rs[t * D + i] = bf16_bits_to_float(qb[t]);
    __syncthreads();
    for (int t = 0; t < nt; t += 2) {
      const float* u = rs + t * D;
      const float* v = rs + min(t + 1, NT - 1) * D;
      float au[4] = {0.0f, 0.0f, 0.0f, 0.0f}, av[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k4 = 0; k4 < D / 4; ++k4)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          au[j] = fmaf(r[k4][j], u[4 * k4 + j], au[j]);
          av[j] = fmaf(r[k4][j], v[4 * k4 + j], av[j]);
        }
      p.qrot[((b0 + t) * p.Hq + h) * D + i] = (au[0] + au[1]) + (au[2] + au[3]);
      if (t + 1 < nt) p.qrot[((b0 + t + 1) * p.Hq + h) * D + i] = (av[0] + av[1]) + (av[2] + av[3]);
    }
  }
}

hipError_t launch_decode_qrot(const AttnParams& p, int D, hipStream_t stream) {
  if (!p.rot) return hipSuccess;
  if (D == 64) {
    if (p.Tq == 1)
      hipLaunchKernelGGL((qrot_kernel<64, 1>), dim3(p.Hq, 1, p.B), dim3(64), 0, stream, p);
    else
      hipLaunchKernelGGL((qrot_kernel<64, kQrotTokens>), dim3(p.Hq, (p.Tq + kQrotTokens - 1) / kQrotTokens, p.B),
                         dim3(64), 0, stream, p);
  } else if (p.Tq == 1)
    hipLaunchKernelGGL((qrot_kernel<128, 1>), dim3(p.Hq, 1, p.B), dim3(128), 0, stream, p);
  else
    hipLaunchKernelGGL((qrot_kernel<128, kQrotTokens>), dim3(p.Hq, (p.Tq + kQrotTokens - 1) / kQrotTokens, p.B),
                       dim3(128), 0, stream, p);
  return hipGetLastError();
}

template <int D>
static void launch_split_w(const AttnParams& p, dim3 grid, hipStream_t stream) {
  if (p.exact_nt)
    hipLaunchKernelGGL(exact_decode_kernel<D>, grid, dim3(kThreads), 0, stream, p);
  else if (p.qw == 2)
    hipLaunchKernelGGL((split_decode_kernel<D, 2>), grid, dim3(kThreads), 0, stream, p);
  else if (p.qw == 3)
    hipLaunchKernelGGL((split_decode_kernel<D, 3>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((split_decode_kernel<D, 4>), grid, dim3(kThreads), 0, stream, p);
}

// Workgroups are handed to the 8 XCDs round-robin in linear id order, and a
// unit's (sequence, kv head) splits have consecutive ids: with an even split
// count in a batch of sequences every unit would start on the same XCDs,
// which then take all the low-index splits (the ones the short sequences of
// a ragged batch still have) while others idle.  There each unit's splits
// are rotated by its index (a bijection, so no workgroup is added).  A
// single sequence keeps the plain order: its units are alike.
hipError_t launch_decode(const AttnParams& p0, int D, hipStream_t stream) {
  AttnParams p = p0;
  p.split_rotate = p.B > 1 && ((p.Sq + p.Se) & 1) == 0;
  dim3 grid(p.Sq + p.Se, p.Hkv, p.B);
  hipError_t e = launch_decode_qrot(p, D, stream);
  if (e != hipSuccess) return e;
  if (D == 64) {
    launch_split_w<64>(p, grid, stream);
    launch_merge_d<64>(p, stream);
  } else {
    launch_split_w<128>(p, grid, stream);
    launch_merge_d<128>(p, stream);
  }
  return hipGetLastError();
}

// The split kernel alone on a grid of (splits, Hkv, sequences), and the merge
// alone (a staged decode launches the split kernel per staged chunk).
hipError_t launch_decode_splits(const AttnParams& p, int D, int splits, int seqs, hipStream_t stream) {
  dim3 grid(splits, p.Hkv, seqs);
  if (D == 64)
    launch_split_w<64>(p, grid, stream);
  else
    launch_split_w<128>(p, grid, stream);
  return hipGetLastError();
}

hipError_t launch_decode_merge(const AttnParams& p, int D, hipStream_t stream) {
  if (D == 64)
    launch_merge_d<64>(p, stream);
  else
    launch_merge_d<128>(p, stream);
  return hipGetLastError();
}

hipError_t launch_lse_merge(const float* op, const float* lp, int P, int R, int d, float* o, float* lse,
                            hipStream_t stream) {
  int threads = d >= 256 ? 256 : ((d + 63) / 64) * 64;
  hipLaunchKernelGGL(lse_merge_kernel, dim3(R), dim3(threads), 0, stream, op, lp, P, R, d, o, lse);
  return hipGetLastError();
}

}  // namespace akv
