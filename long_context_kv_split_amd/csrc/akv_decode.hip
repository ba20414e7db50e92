// Split-KV decode attention over a two-tier history, and the exact
// log-sum-exp merge (ActiveKV, "Context beyond VRAM", "What I built": exact
// and compact tiers merged with exact attention arithmetic; the statistic
// each partial carries is the log-sum-exp added to the paged-attention path in
// "Bringing a serving stack up on new silicon", "What I built").
//
// One workgroup (4 waves) per (split, kv head, sequence).  A split is a fixed
// run of P tokens of one tier; the waves take its 64-token blocks round-robin
// and stream them in 32-token halves.  The G <= 8 query heads sharing the kv
// head are the columns of 16x16x32 matrix-core tiles:
//   scores:  D[token][col] = K_tile[token][dims] x Q[dims][col]
//   values:  O^T[dim][col] += V^T[dim][tokens] x P^T[tokens][col]
// Compressed tier (QuantForge walkthrough, section 1: the query is rotated
// once instead of inverse-rotating blocks): the query is rotated by the
// Walsh-Hadamard butterflies in fp32 and split into fp16 hi + lo halves
// occupying columns 0..7 and 8..15, so the score keeps ~fp32 precision;
// K codes are expanded through an LDS table into fp16 hi and lo parts of the
// Lloyd-Max levels (two tiles per group), the fp16 group scale is applied to
// the fp32 group partial score; V codes are expanded to fp16 level x scale.
// The value sum stays in rotated space; the merge kernel inverse-rotates it.
// Exact tier: bf16 K and q go straight into bf16 tiles (exact products);
// V is staged in LDS to form the transposed operand.
// Each wave keeps an online softmax (base-2, running max and sum); the four
// waves merge in a fixed order, so repeated runs are bit-identical.
#include "akv_common.h"
#include "akv_params.h"

namespace akv {



constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLdsBytes = 65536;
constexpr int kVPitch = 260;  // bytes per staged exact-tier V row (bank spread)

__device__ inline float4v mfma16(half8 a, half8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ inline float4v mfma16bf(bf16x8 a, bf16x8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// value of lane (l ^ 8) within each row of 16 lanes
__device__ inline float row_swap8(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF, 0xF, true));
}

__device__ inline half2v u32_as_h2(uint32_t x) { return __builtin_bit_cast(half2v, x); }
__device__ inline uint32_t h2_as_u32(half2v x) { return __builtin_bit_cast(uint32_t, x); }

struct SoftmaxState {
  float m;  // running max (log2 units)
  float l;  // this lane's share of the running sum
};

// Online-softmax step on 8 scores of one head held by this lane; the running
// max is shared by the 4 lanes (rows 0..3 of 16) with the same column.
__device__ inline float softmax_step(SoftmaxState& st, float (&s)[8], float (&p)[8]) {
  float mx = s[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) mx = fmaxf(mx, s[e]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  float mnew = fmaxf(st.m, mx);
  float muse = (mnew == neg_inf()) ? 0.0f : mnew;
  float alpha = __builtin_amdgcn_exp2f(st.m - muse);
  float sum = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = __builtin_amdgcn_exp2f(s[e] - muse);
    sum += p[e];
  }
  st.l = st.l * alpha + sum;
  st.m = mnew;
  return alpha;
}

// ------------------------------------------------------------------ epilogue
// Merge the 4 waves' (m, l, O) of this workgroup and write the split partial.
template <int D>
__device__ void split_epilogue(const AttnParams& p, unsigned char* smem, int b, int kv, int sx,
                               const SoftmaxState& st, const float4v (&O)[D / 16], bool poison) {
  constexpr int NT = D / 16;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j = lane & 15, qq = lane >> 4;
  float* sm_m = reinterpret_cast<float*>(smem);           // [4][8]
  float* sm_l = sm_m + kWaves * 8;                         // [4][8]
  int* sm_bad = reinterpret_cast<int*>(sm_l + kWaves * 8); // [4]
  float* sm_o = reinterpret_cast<float*>(smem + 512);      // [4][8][D]
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  __syncthreads();  // everyone is done with the LUT / staging region
  if (j < 8) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm_o[(w * 8 + j) * D + 16 * t + 4 * qq + r] = O[t][r];
    if (qq == 0) {
      sm_m[w * 8 + j] = st.m;
      sm_l[w * 8 + j] = l;
    }
  }
  if (lane == 0) sm_bad[w] = poison ? 1 : 0;
  __syncthreads();
  const int G = p.G, S = p.Sq + p.Se;
  const bool bad = sm_bad[0] | sm_bad[1] | sm_bad[2] | sm_bad[3];
  const size_t prow = ((size_t)(b * p.Hkv + kv) * S + sx) * G;  // Tq = 1
  for (int idx = tid; idx < G * D; idx += kThreads) {
    int g = idx / D, t = idx - g * D;
    float M = neg_inf();
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, sm_m[v * 8 + g]);
    float o, lse;
    if (bad) {
      o = __builtin_nanf("");
      lse = o;
    } else if (M == neg_inf()) {
      o = 0.0f;
      lse = neg_inf();
    } else {
      float L = 0.0f, acc = 0.0f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        float wv = __builtin_amdgcn_exp2f(sm_m[v * 8 + g] - M);
        L += wv * sm_l[v * 8 + g];
        acc += wv * sm_o[(v * 8 + g) * D + t];
      }
      o = acc / L;
      lse = (M + __builtin_log2f(L)) * kLn2;
    }
    p.part_o[(prow + g) * D + t] = o;
    if (t == 0) p.part_lse[prow + g] = lse;
  }
}

// ------------------------------------------------------------- quant tier
template <int D>
__device__ void quant_split(const AttnParams& p, unsigned char* smem, int b, int kv, int sx, int start,
                            int end) {
  constexpr int M = D / 32;   // groups = score tiles per token tile
  constexpr int NT = D / 16;  // value tiles
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j = lane & 15, qq = lane >> 4;
  const int G = p.G;

  // --- rotated, pre-scaled query in LDS: q' = H q * (RN(1/sqrt d) * scale * log2 e)
  float* qf = reinterpret_cast<float*>(smem);
  const uint16_t* qsrc = p.q + ((size_t)b * p.Hq + kv * G) * D;
  for (int i = tid; i < G * D; i += kThreads) qf[i] = bf16_bits_to_float(qsrc[i]);
  __syncthreads();
  for (int h = 1; h < D; h <<= 1) {
    for (int i = tid; i < G * D / 2; i += kThreads) {
      int g = i / (D / 2), r = i - g * (D / 2);
      int lo = ((r & ~(h - 1)) << 1) | (r & (h - 1));
      float a = qf[g * D + lo], c = qf[g * D + lo + h];
      qf[g * D + lo] = a + c;
      qf[g * D + lo + h] = a - c;
    }
    __syncthreads();
  }
  const float qmul = inv_sqrt_d(D) * p.qscale2;
  half8 Q[M];
  {
    const int hj = j & 7;
    const bool lopart = j >= 8;
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = hj < G ? qf[hj * D + 32 * m + 8 * qq + e] * qmul : 0.0f;
        _Float16 hi = (_Float16)v;
        _Float16 lo = (_Float16)(v - (float)hi);
        Q[m][e] = lopart ? lo : hi;
      }
  }
  __syncthreads();

  // --- level table: row e (code byte) = 256 B: 16 x (hi pair, lo pair) | 32 x hi pair
  {
    const int e = tid;  // 256 threads, 256 rows
    float c0 = __builtin_bit_cast(float, kLevelBits[e & 15]);
    float c1 = __builtin_bit_cast(float, kLevelBits[e >> 4]);
    _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
    _Float16 l0 = (_Float16)(c0 - (float)h0), l1 = (_Float16)(c1 - (float)h1);
    uint32_t hip = h2_as_u32(half2v{h0, h1});
    uint32_t lop = h2_as_u32(half2v{l0, l1});
    uint32_t* row = reinterpret_cast<uint32_t*>(smem) + e * 64;
    for (int k = 0; k < 64; ++k) {
      int slot = (k + e) & 63;
      row[slot] = (slot < 32 && (slot & 1)) ? lop : hip;
    }
  }
  __syncthreads();
  const unsigned char* lut = smem;
  const int koff = 8 * j;                 // K copy of this lane
  const int voff = 128 + 4 * (lane & 31); // V copy of this lane

  SoftmaxState st{neg_inf(), 0.0f};
  float4v O[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) O[t] = float4v{0, 0, 0, 0};
  bool poison = false;

  const int blk0 = start >> 6;
  const int nblk = ((end + 63) >> 6) - blk0;
  const int* table = p.qtab + (size_t)b * p.qmax;
  for (int i = w; i < nblk; i += kWaves) {
    const int blk = blk0 + i;
    const int pb = table[blk];
    if (pb < 0 || pb >= p.qnb) {
      poison = true;
      continue;
    }
    const size_t slab = (size_t)pb * p.Hkv + kv;
    const unsigned char* kcs = p.kc + slab * (32 * D);
    const unsigned char* vcs = p.vc + slab * (32 * D);
    const uint16_t* kss = p.ks + slab * (2 * D);
    const uint16_t* vss = p.vs + slab * (2 * D);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int tb = blk * 64 + 32 * c;  // first tier token of this half
      if (tb >= end) break;
      // ---- loads
      uint32_t kw[2][M];
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        int row = 32 * c + 8 * (j >> 2) + 4 * tp + (j & 3);
        const uint32_t* src = reinterpret_cast<const uint32_t*>(kcs + row * (D / 2) + (D / 8) * qq);
        if constexpr (M == 4) {
          u32x4 x = *reinterpret_cast<const u32x4*>(src);
          kw[tp][0] = x[0]; kw[tp][1] = x[1]; kw[tp][2] = x[2]; kw[tp][3] = x[3];
        } else {
          u32x2 x = *reinterpret_cast<const u32x2*>(src);
          kw[tp][0] = x[0]; kw[tp][1] = x[1];
        }
      }
      u32x4 ksc[M], vsc[M];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        ksc[m] = *reinterpret_cast<const u32x4*>(kss + m * 64 + 32 * c + 8 * qq);
        vsc[m] = *reinterpret_cast<const u32x4*>(vss + m * 64 + 32 * c + 8 * qq);
      }
      uint32_t vw[NT];
      {
        const u32x4* src = reinterpret_cast<const u32x4*>(vcs + ((c * 4 + qq) * 16 + j) * (D / 4));
#pragma unroll
        for (int v = 0; v < NT / 4; ++v) {
          u32x4 x = src[v];
          vw[4 * v] = x[0]; vw[4 * v + 1] = x[1]; vw[4 * v + 2] = x[2]; vw[4 * v + 3] = x[3];
        }
      }
      const int nvalid = end - tb;  // tokens of this half that exist (may exceed 32)
      if (nvalid < 32) {
        // zero the value scales of missing tokens so 0 * garbage cannot appear
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) {
            int t0 = 8 * qq + 2 * q2;
            uint32_t x = vsc[m][q2];
            if (t0 >= nvalid) x = 0;
            else if (t0 + 1 >= nvalid) x &= 0xFFFFu;
            vsc[m][q2] = x;
          }
      }
      // ---- scores
      float s[8];
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        float acc[4] = {0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < M; ++m) {
          half8 khi, klo;
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            uint32_t e = (kw[tp][m] >> (8 * bb)) & 0xFFu;
            u32x2 pr = *reinterpret_cast<const u32x2*>(lut + e * 256 + koff);
            half2v h = u32_as_h2(pr[0]), l = u32_as_h2(pr[1]);
            khi[2 * bb] = h[0]; khi[2 * bb + 1] = h[1];
            klo[2 * bb] = l[0]; klo[2 * bb + 1] = l[1];
          }
          float4v dm = mfma16(khi, Q[m], float4v{0, 0, 0, 0});
          dm = mfma16(klo, Q[m], dm);
          // group scales of this lane's rows: tokens 8qq + 4tp + r (r = 0..3)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            int e2 = 4 * tp + r;
            half2v sp = u32_as_h2(ksc[m][e2 >> 1]);
            float sc = (float)sp[e2 & 1];
            acc[r] = fmaf(sc, dm[r], acc[r]);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) s[4 * tp + r] = acc[r];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s[e] += row_swap8(s[e]);  // hi-column + lo-column partial scores
        if (8 * qq + e >= nvalid) s[e] = neg_inf();
      }
      float pr[8];
      float alpha = softmax_step(st, s, pr);
#pragma unroll
      for (int t = 0; t < NT; ++t) O[t] *= alpha;
      half8 pb8;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb8[e] = (_Float16)pr[e];
      // ---- values: V'^T[dim][token] = C16[code] * scale
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int g = t >> 1;
        half8 a;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          uint32_t e = (vw[t] >> (8 * bb)) & 0xFFu;
          half2v lv = u32_as_h2(*reinterpret_cast<const uint32_t*>(lut + e * 256 + voff));
          half2v sv = u32_as_h2(vsc[g][bb]);
          half2v x = lv * sv;
          a[2 * bb] = x[0]; a[2 * bb + 1] = x[1];
        }
        O[t] = mfma16(a, pb8, O[t]);
      }
    }
  }
  split_epilogue<D>(p, smem, b, kv, sx, st, O, poison);
}

// ------------------------------------------------------------- exact tier
template <int D>
__device__ void exact_split(const AttnParams& p, unsigned char* smem, int b, int kv, int sx, int start,
                            int end) {
  constexpr int MK = D / 32;  // score tiles per token tile
  constexpr int NT = D / 16;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j = lane & 15, qq = lane >> 4;
  const int G = p.G;

  // query operand: lane (col j, qq) holds dims qq*D/4 + 8m + e of head j
  bf16x8 Q[MK];
  {
    const int hj = min(j, G - 1);  // padded columns read a valid head, then zero
    const uint16_t* qsrc = p.q + ((size_t)b * p.Hq + kv * G + hj) * D + qq * (D / 4);
#pragma unroll
    for (int m = 0; m < MK; ++m) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qsrc + 8 * m);
      if (j >= G) x = u32x4{0, 0, 0, 0};
      Q[m] = __builtin_bit_cast(bf16x8, x);
    }
  }
  unsigned char* vst = smem + w * (32 * kVPitch + 64);  // this wave's V staging rows

  SoftmaxState st{neg_inf(), 0.0f};
  float4v O[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) O[t] = float4v{0, 0, 0, 0};
  bool poison = false;

  const int blk0 = start >> 6;
  const int nblk = ((end + 63) >> 6) - blk0;
  const int* table = p.etab + (size_t)b * p.emax;
  for (int i = w; i < nblk; i += kWaves) {
    const int blk = blk0 + i;
    const int pb = table[blk];
    if (pb < 0 || pb >= p.enb) {
      poison = true;
      continue;
    }
    const uint16_t* kslab = p.ek + ((size_t)pb * p.Hkv + kv) * kBlock * D;
    const uint16_t* vslab = p.ev + ((size_t)pb * p.Hkv + kv) * kBlock * D;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int tb = blk * 64 + 32 * c;
      if (tb >= end) break;
      const int nvalid = end - tb;
      // ---- loads: K rows of both tiles; V half (32 rows)
      u32x4 kx[2][MK];
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        int row = 32 * c + 8 * (j >> 2) + 4 * tp + (j & 3);
        const u32x4* src = reinterpret_cast<const u32x4*>(kslab + row * D + qq * (D / 4));
#pragma unroll
        for (int m = 0; m < MK; ++m) kx[tp][m] = src[m];
      }
      constexpr int CH = D / 8;             // 16-byte chunks per row
      constexpr int PER = 32 * CH / 64;     // chunks per lane
      u32x4 vx[PER];
      const u32x4* vsrc = reinterpret_cast<const u32x4*>(vslab + 32 * c * D);
#pragma unroll
      for (int k = 0; k < PER; ++k) vx[k] = vsrc[lane + 64 * k];
      // ---- stage V rows (zeros for missing tokens); LDS ops of one wave run in order
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        int ci = lane + 64 * k, row = ci / CH, col = ci - row * CH;
        u32x4 x = (row < nvalid) ? vx[k] : u32x4{0, 0, 0, 0};
        uint32_t* dst = reinterpret_cast<uint32_t*>(vst + row * kVPitch + col * 16);
        dst[0] = x[0]; dst[1] = x[1]; dst[2] = x[2]; dst[3] = x[3];
      }
      __builtin_amdgcn_wave_barrier();
      // ---- scores
      float s[8];
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        float4v dm = float4v{0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < MK; ++m) dm = mfma16bf(__builtin_bit_cast(bf16x8, kx[tp][m]), Q[m], dm);
#pragma unroll
        for (int r = 0; r < 4; ++r) s[4 * tp + r] = dm[r] * p.qscale2;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (8 * qq + e >= nvalid) s[e] = neg_inf();
      float pr[8];
      float alpha = softmax_step(st, s, pr);
#pragma unroll
      for (int t = 0; t < NT; ++t) O[t] *= alpha;
      bf16x8 pb8;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb8[e] = (__bf16)pr[e];
      // ---- values: V^T[dim 16t + j][token 8qq + e] from the staged rows
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        bf16x8 a;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          a[e] = *reinterpret_cast<const __bf16*>(vst + (8 * qq + e) * kVPitch + (16 * t + j) * 2);
        O[t] = mfma16bf(a, pb8, O[t]);
      }
    }
  }
  split_epilogue<D>(p, smem, b, kv, sx, st, O, poison);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void split_decode_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];
  const int sx = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const bool quant = sx < p.Sq;
  const int s = quant ? sx : sx - p.Sq;
  const int P = quant ? p.Pq : p.Pe;
  const int maxb = quant ? p.qmax : p.emax;
  const int len = maxb ? (quant ? p.qlen[b] : p.elen[b]) : 0;
  if (len < 0 || len > maxb * 64) return;  // merge reports the sequence as NaN
  const int start = s * P;
  if (start >= len) return;
  const int end = min(start + P, len);
  if (quant)
    quant_split<D>(p, smem, b, kv, sx, start, end);
  else
    exact_split<D>(p, smem, b, kv, sx, start, end);
}

// --------------------------------------------------------------- merging
// Merge partials [first, first + n) (stride in partial rows) of one row in
// ascending order; returns this thread's output element and the row lse.
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
  o = (wa / W) * oa + (wb / W) * ob;
  lse = M + __logf(W);
}

template <int D>
__global__ __launch_bounds__(D) void merge_kernel(AttnParams p) {
  __shared__ float buf[D];
  const int row = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int tau = row / p.Hq, h = row - tau * p.Hq;
  const int G = p.G, kv = h / G, g = h - kv * G;
  const int S = p.Sq + p.Se;
  const int ql = p.qmax ? p.qlen[b] : 0;
  const int el = p.emax ? p.elen[b] : 0;
  float* out = p.o + (((size_t)b * p.Tq + tau) * p.Hq + h) * D;
  float* lout = p.lse + ((size_t)b * p.Tq + tau) * p.Hq + h;
  if (ql < 0 || ql > 64 * p.qmax || el < 0 || el > 64 * p.emax) {
    out[t] = __builtin_nanf("");
    if (t == 0) *lout = __builtin_nanf("");
    return;
  }
  const int nq = (ql + p.Pq - 1) / p.Pq, ne = (el + p.Pe - 1) / p.Pe;
  const size_t stride = (size_t)p.Tq * G;                               // partial rows per split
  const size_t base = ((size_t)(b * p.Hkv + kv) * S) * stride + (size_t)tau * G + g;
  // (i) compressed-tier partials, rotated space
  float oq, lq;
  merge_run(p.part_o, p.part_lse, base, stride, nq, D, t, oq, lq);
  // (ii) inverse rotation once per head: o = (H o_rot) * RN(1/sqrt d)
  buf[t] = oq;
  __syncthreads();
  for (int hh = 1; hh < D; hh <<= 1) {
    float a = buf[t], c = buf[t ^ hh];
    __syncthreads();
    buf[t] = (t & hh) ? (c - a) : (a + c);
    __syncthreads();
  }
  oq = buf[t] * inv_sqrt_d(D);
  // (iii) exact-tier partials
  float oe, le;
  merge_run(p.part_o, p.part_lse, base + (size_t)p.Sq * stride, stride, ne, D, t, oe, le);
  // (iv) both tiers
  float o, lse;
  merge_two(oq, lq, oe, le, o, lse);
  out[t] = o;
  if (t == 0) *lout = lse;
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

hipError_t launch_decode(const AttnParams& p, int D, hipStream_t stream) {
  dim3 grid(p.Sq + p.Se, p.Hkv, p.B);
  dim3 mgrid(p.Tq * p.Hq, p.B);
  if (D == 64) {
    hipLaunchKernelGGL(split_decode_kernel<64>, grid, dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL(merge_kernel<64>, mgrid, dim3(64), 0, stream, p);
  } else {
    hipLaunchKernelGGL(split_decode_kernel<128>, grid, dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL(merge_kernel<128>, mgrid, dim3(128), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_lse_merge(const float* op, const float* lp, int P, int R, int d, float* o, float* lse,
                            hipStream_t stream) {
  int threads = d >= 256 ? 256 : ((d + 63) / 64) * 64;
  hipLaunchKernelGGL(lse_merge_kernel, dim3(R), dim3(threads), 0, stream, op, lp, P, R, d, o, lse);
  return hipGetLastError();
}

}  // namespace akv
