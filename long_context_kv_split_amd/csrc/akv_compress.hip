// Compress evicted exact-tier tokens into the 4-bit tier.
//
// For every (token, kv head, K|V) vector of d bf16 values (ActiveKV, "Context
// beyond VRAM", "What I built": tokens leaving the recent window are encoded
// into the small tier; the rotation is the Walsh-Hadamard rotation of the
// QuantForge walkthrough, section 1):
//   E1 x = float(bf16)                                   exact
//   E2 unnormalized Sylvester butterflies, h = 1, 2, ..., d/2 ascending:
//      (x[i], x[i+h]) <- (x[i] + x[i+h], x[i] - x[i+h])  for i & h == 0
//   E3 y = x * RN(1/sqrt(d))
//   E4 per 32-group: sq = y*y, pairwise tree (off = 16, 8, 4, 2, 1:
//      v[i] += v[i+off]), ms = sum / 32, s32 = sqrt(ms) (correctly rounded)
//   E5 s16 = fp16 round-to-nearest-even (saturating at 65504) -- the stored scale
//   E6 s = float(s16); s == 0 -> every code of the group is 7
//   E7 u = y / s (correctly rounded)
//   E8 code = #{k : u > T_k}   (nearest Lloyd-Max level, ties to lower index)
//   E9 two codes per byte, storage order as documented in akv.h
// Every step is one IEEE float32 operation with round-to-nearest-even and
// nothing is contracted into a fused multiply-add, so codes and scales are
// bit-exact functions of the input.
//
// With a given orthogonal rotation R (the QuantForge walkthrough, section 5,
// compares a QR rotation with the Hadamard one), E2 is y = R x summed in
// ascending k and E3 is dropped.
//
// One wavefront per (destination token pair, kv head, K|V) -- per 8 pairs with
// a given rotation, which then share each load of R: lane l holds elements
// l + 64k; butterflies with h < 64 exchange across lanes.  Destination pairs
// are aligned to the compressed tier's positions (2q, 2q + 1), because two
// tokens share each value-code byte: when the range starts at an odd position
// the first pair holds one token already there, and a pair's byte is read,
// merged and written back by its one wavefront, so every byte has one writer
// and the bits of positions outside the range keep their value.
#include "akv_common.h"

#pragma clang fp contract(off)

namespace akv {

struct CompressParams {
  int Hkv;
  const uint16_t* src_k;
  const uint16_t* src_v;
  const int32_t* src_table;
  int src_num_blocks, src_start, n_tokens;
  uint8_t* dst_kc;
  uint8_t* dst_vc;
  uint16_t* dst_ks;
  uint16_t* dst_vs;
  const int32_t* dst_table;
  int dst_num_blocks, dst_start;
  const float* rot;  // nullptr: Walsh-Hadamard; else float32 [d][d] orthogonal R
};

// E1 for token `tok` of the range (lane l takes elements l + 64k): zeros, and
// false, past the range or for a block id outside the pool.  Exact-tier K is
// token-major (a token's dims adjacent), V dim-major inside each 32-token
// half block (dim t of token r at ((r / 32) * d + t) * 32 + r % 32).
template <int D>
__device__ inline bool load_token(const CompressParams& p, int isv, int kv, int tok, int lane, float (&x)[D / 64]) {
  constexpr int E = D / 64;
  const uint16_t* src = nullptr;
  const int dstride = isv ? kBlock / 2 : 1;
  if (tok >= 0 && tok < p.n_tokens) {
    const int s = p.src_start + tok;
    const int blk = p.src_table[s >> 6];
    if (blk >= 0 && blk < p.src_num_blocks) {
      const size_t slab = (size_t)(blk * p.Hkv + kv) * kBlock * D;
      src = isv ? p.src_v + slab + ((s & 63) >> 5) * (kBlock / 2) * D + (s & 31) : p.src_k + slab + (size_t)(s & 63) * D;
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = src ? bf16_bits_to_float(src[(lane + 64 * e) * dstride]) : 0.0f;
  return src != nullptr;
}

// E2, Walsh-Hadamard: butterflies across lanes for h < 64, inside the lane
// for h = 64.
template <int D>
__device__ inline void hadamard_rows(float (&x)[D / 64], int lane) {
  constexpr int E = D / 64;
#pragma unroll
  for (int h = 1; h < 64 && h < D; h <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float o = __shfl_xor(x[e], h);
      x[e] = (lane & h) ? (o - x[e]) : (x[e] + o);
    }
  }
  if (E == 2) {
    float a = x[0], b = x[E - 1];
    x[0] = a + b;
    x[E - 1] = a - b;
  }
}

// E2 with a given rotation R for NT tokens at once: y_i = (((0 + R_i0 x_0) +
// R_i1 x_1) + ...), ascending k, one float32 multiply and one add per term
// (no E3).  Lane l computes rows i = l + 64e; each float4 of R it loads
// serves all NT tokens, whose values are broadcast from LDS (xs: NT * D
// floats, this wavefront's own).
template <int D, int NT>
__device__ inline void dense_rows(const float* __restrict__ R, float (&x)[NT][D / 64], int lane, float* xs) {
  constexpr int E = D / 64;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < E; ++e) xs[t * D + lane + 64 * e] = x[t][e];
  __syncthreads();
  float acc[NT][E];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[t][e] = 0.0f;
  for (int k4 = 0; k4 < D / 4; ++k4) {
    float4v r[E];
#pragma unroll
    for (int e = 0; e < E; ++e) r[e] = *reinterpret_cast<const float4v*>(R + (size_t)(lane + 64 * e) * D + 4 * k4);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float4v xv = *reinterpret_cast<const float4v*>(xs + t * D + 4 * k4);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[t][e] = acc[t][e] + r[e][u] * xv[u];
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < E; ++e) x[t][e] = acc[t][e];
}

// E9 at code width W < 4 (the pair plane, then for W = 3 the high plane; the
// layouts are those of include/akv.h): the pair's codes go to LDS (0 for a
// missing token), then each lane assembles whole output bytes.  K rows of
// missing tokens are not written; a V byte always is.
template <int D, int W>
__device__ inline void store_narrow(const CompressParams& p, size_t slab, int r0, const bool (&ours)[2], int isv,
                                    int lane, const int (&code)[2][D / 64], const bool (&ok)[2], unsigned char* cs) {
  constexpr int E = D / 64, M = D / 32;
  __syncthreads();  // the previous pair's reads of cs are done
#pragma unroll
  for (int tk = 0; tk < 2; ++tk)
#pragma unroll
    for (int e = 0; e < E; ++e) cs[tk * D + lane + 64 * e] = (ours[tk] && ok[tk]) ? (unsigned char)code[tk][e] : 0;
  __syncthreads();
  if (!isv) {
    uint8_t* kslab = p.dst_kc + slab * (8 * W * D);
    for (int tk = 0; tk < 2; ++tk) {
      if (!(ours[tk] && ok[tk])) continue;
      const unsigned char* ct = cs + tk * D;
      if (lane < D / 4) {  // pair plane: byte (d/16) a + 4 n + b of the row
        const int a = lane / (D / 16), r = lane % (D / 16), n = r >> 2, b = r & 3;
        int byte = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 2; ++e) byte |= (ct[32 * (2 * n + h) + 8 * a + 2 * b + e] & 3) << (4 * h + 2 * e);
        kslab[(r0 + tk) * (D / 4) + lane] = (uint8_t)byte;
      }
      if (W == 3 && lane < D / 8) {  // high plane: row bit 8Ma + 2Mb + 2m + e
        const int a = lane / M, q = lane % M;
        int byte = 0;
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
          const int g = 8 * q + bit, b = g / (2 * M), rem = g % (2 * M), m = rem >> 1, e = rem & 1;
          byte |= ((ct[32 * m + 8 * a + 2 * b + e] >> 2) & 1) << bit;
        }
        kslab[16 * D + (r0 + tk) * (D / 8) + lane] = (uint8_t)byte;
      }
    }
  } else {
    // a byte holds bits of both tokens of the pair; those of a position
    // outside the range are kept (pair plane: bits 2e, 2e + 1, 4 + 2e,
    // 5 + 2e of token e; high plane: bits 2h + e)
    uint8_t* vslab = p.dst_vc + slab * (8 * W * D);
    const int c = r0 >> 5, a = (r0 >> 3) & 3, b = (r0 >> 1) & 3;
    const int keep2 = (ours[0] ? 0 : 0x33) | (ours[1] ? 0 : 0xCC);
    const int keep1 = (ours[0] ? 0 : 0x55) | (ours[1] ? 0 : 0xAA);
    for (int l = lane; l < D / 2; l += 64) {  // pair plane: dim 16(2n + h) + i
      const int i = l & 15, n = l >> 4;
      int byte = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 2; ++e) byte |= (cs[e * D + 16 * (2 * n + h) + i] & 3) << (4 * h + 2 * e);
      uint8_t* dst = vslab + ((c * 4 + a) * 16 + i) * (D / 8) + 4 * n + b;
      if (keep2) byte = (byte & ~keep2) | (*dst & keep2);
      *dst = (uint8_t)byte;
    }
    if (W == 3) {
      for (int l = lane; l < D / 4; l += 64) {  // high plane: dim 16(4n + h) + i
        const int i = l & 15, n = l >> 4;
        int byte = 0;
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
          for (int e = 0; e < 2; ++e) byte |= ((cs[e * D + 16 * (4 * n + h) + i] >> 2) & 1) << (2 * h + e);
        uint8_t* dst = vslab + 16 * D + ((c * 4 + a) * 16 + i) * (D / 16) + 4 * n + b;
        if (keep1) byte = (byte & ~keep1) | (*dst & keep1);
        *dst = (uint8_t)byte;
      }
    }
  }
}

// Source token (index in the range) of slot tk of destination pair `pair`:
// the pair covers compressed positions (dst_start & ~1) + 2 pair + {0, 1}.
__device__ inline int pair_token(const CompressParams& p, int pair, int tk) {
  return 2 * pair + tk - (p.dst_start & 1);
}

// E4..E9 for destination pair `pair` of one (kv head, K|V), given its rotated
// values y (lane l: elements l + 64k), at code width W (cs: 2 * D bytes of
// LDS, this wavefront's own).  A slot whose position is outside the range is
// not ours: nothing of it is written, and its half of the value byte is kept.
template <int D, int W>
__device__ inline void finish_pair(const CompressParams& p, int pair, int kv, int isv, int lane,
                                   const float (&y)[2][D / 64], const bool (&ok)[2], unsigned char* cs) {
  constexpr int E = D / 64;
  bool ours[2];
#pragma unroll
  for (int tk = 0; tk < 2; ++tk) {
    const int t = pair_token(p, pair, tk);
    ours[tk] = t >= 0 && t < p.n_tokens;
  }
  int code[2][E];
  uint16_t s16[2][E];
#pragma unroll
  for (int tk = 0; tk < 2; ++tk) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float v = y[tk][e] * y[tk][e];                        // E4
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) {
        float o = __shfl_down(v, off, 32);
        v = v + o;
      }
      float ms = v * 0.03125f;
      float s32 = __builtin_sqrtf(ms);
      __half hs = __float2half_rn(fminf(s32, 65504.0f));    // E5
      uint16_t hb = __half_as_ushort(hs);
      hb = (uint16_t)__shfl((int)hb, lane & 32);            // broadcast group scale
      s16[tk][e] = hb;
      float s = __half2float(__ushort_as_half(hb));         // E6
      int c = (1 << (W - 1)) - 1;                           // the lower middle level
      if (s != 0.0f) {
        float u = y[tk][e] / s;                             // E7
        c = 0;
#pragma unroll
        for (int k = 0; k < (1 << W) - 1; ++k) c += (u > __builtin_bit_cast(float, thresh_bits<W>()[k])) ? 1 : 0;  // E8
      }
      code[tk][e] = c;
    }
  }

  // E9: store
  const int pos0 = (p.dst_start & ~1) + 2 * pair;   // even
  const int dblk = p.dst_table[pos0 >> 6];
  if (dblk < 0 || dblk >= p.dst_num_blocks) return;
  const int r0 = pos0 & 63;
  const size_t slab = (size_t)dblk * p.Hkv + kv;
  uint16_t* scales = (isv ? p.dst_vs : p.dst_ks) + slab * (2 * D);
  if constexpr (W < 4) {
    store_narrow<D, W>(p, slab, r0, ours, isv, lane, code, ok, cs);
#pragma unroll
    for (int tk = 0; tk < 2; ++tk)
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (ours[tk] && ok[tk] && (lane & 31) == 0) scales[((lane + 64 * e) >> 5) * kBlock + r0 + tk] = s16[tk][e];
    return;
  }
  if (!isv) {
    uint8_t* codes = p.dst_kc + slab * (32 * D);
#pragma unroll
    for (int tk = 0; tk < 2; ++tk) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        int hi = __shfl_down(code[tk][e], 1);
        int dim = lane + 64 * e;
        if (ours[tk] && ok[tk] && !(lane & 1))
          codes[(r0 + tk) * (D / 2) + kcode_byte(D, dim)] = (uint8_t)(code[tk][e] | (hi << 4));
        if (ours[tk] && ok[tk] && (lane & 31) == 0)
          scales[(dim >> 5) * kBlock + r0 + tk] = s16[tk][e];
      }
    }
  } else {
    uint8_t* codes = p.dst_vc + slab * (32 * D);
    // the nibble of a position outside the range is kept
    const int keep = (ours[0] ? 0 : 0x0F) | (ours[1] ? 0 : 0xF0);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      int dim = lane + 64 * e;
      int c0 = (ours[0] && ok[0]) ? code[0][e] : 0;
      int c1 = (ours[1] && ok[1]) ? code[1][e] : 0;
      uint8_t* dst = codes + vcode_byte(D, r0, dim);
      int byte = c0 | (c1 << 4);
      if (keep) byte = (byte & ~keep) | (*dst & keep);
      *dst = (uint8_t)byte;
#pragma unroll
      for (int tk = 0; tk < 2; ++tk)
        if (ours[tk] && ok[tk] && (lane & 31) == 0) scales[(dim >> 5) * kBlock + r0 + tk] = s16[tk][e];
    }
  }
}

// Encode destination pairs pair0 .. pair0 + NP - 1 of one (kv head, K|V): one
// wavefront, lane l holding elements l + 64k.  With a given rotation the NP
// pairs share the loads of R (xs: 2 * NP * D floats of LDS).
template <int D, int NP, int W>
__device__ inline void encode_pairs(const CompressParams& p, int pair0, int kv, int isv, int lane, float* xs,
                                    unsigned char* cs) {
  constexpr int E = D / 64;
  const float rd = inv_sqrt_d(D);
  float x[2 * NP][E];
  bool ok[2 * NP];
#pragma unroll
  for (int i = 0; i < 2 * NP; ++i) ok[i] = load_token<D>(p, isv, kv, pair_token(p, pair0, i), lane, x[i]);  // E1
  if (p.rot) {
    dense_rows<D, 2 * NP>(p.rot, x, lane, xs);                                                       // E2
  } else {
#pragma unroll
    for (int i = 0; i < 2 * NP; ++i) hadamard_rows<D>(x[i], lane);                                  // E2
  }
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    if (pair_token(p, pair0 + j, 0) >= p.n_tokens) break;
    float y[2][E];
    const bool okp[2] = {ok[2 * j], ok[2 * j + 1]};
#pragma unroll
    for (int tk = 0; tk < 2; ++tk)
#pragma unroll
      for (int e = 0; e < E; ++e) y[tk][e] = p.rot ? x[2 * j + tk][e] : x[2 * j + tk][e] * rd;       // E3 (Hadamard only)
    finish_pair<D, W>(p, pair0 + j, kv, isv, lane, y, okp, cs);
  }
}

// grid (ceil(pairs / NP), Hkv, K|V), one wavefront each
constexpr int kDensePairs = 8;
template <int D, int NP, int W>
__global__ __launch_bounds__(64) void compress_kernel(CompressParams p) {
  __shared__ __attribute__((aligned(16))) float xs[2 * NP * D];
  __shared__ unsigned char cs[2 * D];
  encode_pairs<D, NP, W>(p, blockIdx.x * NP, blockIdx.y, blockIdx.z, threadIdx.x, xs, cs);
}

// ------------------------------------------------------------ per-step append / evict
struct StepParams {
  int B, Hkv, window;
  const uint16_t* new_k;
  const uint16_t* new_v;
  uint16_t* ek;
  uint16_t* ev;
  int32_t* etab;
  int32_t* elen;
  int emax, enb;
  uint8_t* kc;
  uint8_t* vc;
  uint16_t* ks;
  uint16_t* vs;
  const int32_t* qtab;
  int32_t* qlen;
  int qmax, qnb;
  const float* rot;
};

// What the step does to sequence b, decided from its lengths before the
// step (both kernels of the step take the same decision).
struct StepPlan {
  int n, m;        // exact and compressed lengths before the step
  bool append;     // the new token has a place in the exact table
  bool evict;      // the exact tier's first block moves to the compressed tier
};

__device__ inline StepPlan step_plan(const StepParams& p, int b) {
  StepPlan s;
  s.n = p.elen[b];
  s.m = p.qlen[b];
  s.append = s.n >= 0 && (s.n >> 6) < p.emax;
  s.evict = s.append && s.n + 1 >= p.window + kBlock && s.m >= 0 && s.m + kBlock <= p.qmax * kBlock;
  return s;
}

// grid (34, Hkv, 2B): x < 33 encodes destination pair x of the evicted block
// (when the sequence evicts; 64 tokens at compressed position m take 32 pairs
// for an even m and 33 for an odd one), x == 33 writes the new token;
// z = 2 b + (K|V).  The append writes block n / 64 >= 1 while the encode reads
// block 0, so the two never touch the same bytes.
template <int D, int W>
__global__ __launch_bounds__(64) void append_evict_kernel(StepParams p) {
  __shared__ __attribute__((aligned(16))) float xs[2 * D];
  __shared__ unsigned char cs[2 * D];
  const int x = blockIdx.x, kv = blockIdx.y, b = blockIdx.z >> 1, isv = blockIdx.z & 1, lane = threadIdx.x;
  const StepPlan s = step_plan(p, b);
  if (x == kBlock / 2 + 1) {
    if (!s.append) return;
    const int pb = p.etab[(size_t)b * p.emax + (s.n >> 6)];
    if (pb < 0 || pb >= p.enb) return;  // the attention reports the bad id as NaN
    const int r = s.n & 63;
    const uint16_t* src = (isv ? p.new_v : p.new_k) + ((size_t)b * p.Hkv + kv) * D;
    const size_t slab = ((size_t)pb * p.Hkv + kv) * kBlock * D;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
      const int t = lane + 64 * e;
      if (!isv)
        p.ek[slab + (size_t)r * D + t] = src[t];  // token-major
      else
        p.ev[slab + ((size_t)(r >> 5) * D + t) * (kBlock / 2) + (r & 31)] = src[t];  // dim-major per half block
    }
    return;
  }
  if (!s.evict || x >= (kBlock + 1 + (s.m & 1)) / 2) return;
  CompressParams c;
  c.Hkv = p.Hkv;
  c.src_k = p.ek;
  c.src_v = p.ev;
  c.src_table = p.etab + (size_t)b * p.emax;
  c.src_num_blocks = p.enb;
  c.src_start = 0;
  c.n_tokens = kBlock;
  c.dst_kc = p.kc;
  c.dst_vc = p.vc;
  c.dst_ks = p.ks;
  c.dst_vs = p.vs;
  c.dst_table = p.qtab + (size_t)b * p.qmax;
  c.dst_num_blocks = p.qnb;
  c.dst_start = s.m;
  c.rot = p.rot;
  encode_pairs<D, 1, W>(c, x, kv, isv, lane, xs, cs);
}

// After the encode has read the old first block: lengths, and the rotation
// of the ceil((n + 1) / 64) blocks in use so the freed block comes right after
// the ones still in use.
__global__ __launch_bounds__(64) void step_commit_kernel(StepParams p) {
  const int b = blockIdx.x * 64 + threadIdx.x;
  if (b >= p.B) return;
  const StepPlan s = step_plan(p, b);
  if (!s.append) {
    p.elen[b] = -1;
    return;
  }
  if (!s.evict) {
    p.elen[b] = s.n + 1;
    return;
  }
  int32_t* row = p.etab + (size_t)b * p.emax;
  const int used = (s.n + 1 + kBlock - 1) / kBlock;
  const int first = row[0];
  for (int i = 0; i + 1 < used; ++i) row[i] = row[i + 1];
  row[used - 1] = first;
  p.elen[b] = s.n + 1 - kBlock;
  p.qlen[b] = s.m + kBlock;
}

template <int D, int NP>
void launch_compress_w(int W, dim3 grid, hipStream_t stream, const CompressParams& p) {
  if (W == 2)
    hipLaunchKernelGGL((compress_kernel<D, NP, 2>), grid, dim3(64), 0, stream, p);
  else if (W == 3)
    hipLaunchKernelGGL((compress_kernel<D, NP, 3>), grid, dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL((compress_kernel<D, NP, 4>), grid, dim3(64), 0, stream, p);
}

template <int D>
void launch_append_w(int W, dim3 grid, hipStream_t stream, const StepParams& p) {
  if (W == 2)
    hipLaunchKernelGGL((append_evict_kernel<D, 2>), grid, dim3(64), 0, stream, p);
  else if (W == 3)
    hipLaunchKernelGGL((append_evict_kernel<D, 3>), grid, dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL((append_evict_kernel<D, 4>), grid, dim3(64), 0, stream, p);
}

hipError_t launch_compress(const akv_compress_desc* d, hipStream_t stream) {
  CompressParams p;
  p.Hkv = d->Hkv;
  p.src_k = d->src_k;
  p.src_v = d->src_v;
  p.src_table = d->src_block_table;
  p.src_num_blocks = d->src_num_blocks;
  p.src_start = d->src_start;
  p.n_tokens = d->n_tokens;
  p.dst_kc = d->dst_k_codes;
  p.dst_vc = d->dst_v_codes;
  p.dst_ks = d->dst_k_scales;
  p.dst_vs = d->dst_v_scales;
  p.dst_table = d->dst_block_table;
  p.dst_num_blocks = d->dst_num_blocks;
  p.dst_start = d->dst_start;
  p.rot = d->rotation;
  // destination pairs (aligned to even positions); a given rotation: 8 pairs
  // per wavefront share each load of R
  const int pairs = ((d->dst_start & 1) + d->n_tokens + 1) / 2;
  const int W = code_width(d->code_bits);
  if (p.rot) {
    dim3 grid((pairs + kDensePairs - 1) / kDensePairs, d->Hkv, 2);
    if (d->d == 64)
      launch_compress_w<64, kDensePairs>(W, grid, stream, p);
    else
      launch_compress_w<128, kDensePairs>(W, grid, stream, p);
  } else {
    dim3 grid(pairs, d->Hkv, 2);
    if (d->d == 64)
      launch_compress_w<64, 1>(W, grid, stream, p);
    else
      launch_compress_w<128, 1>(W, grid, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_append_evict(const akv_append_desc* d, hipStream_t stream) {
  StepParams p;
  p.B = d->B;
  p.Hkv = d->Hkv;
  p.window = d->window;
  p.new_k = d->new_k;
  p.new_v = d->new_v;
  p.ek = d->exact_k;
  p.ev = d->exact_v;
  p.etab = d->exact_table;
  p.elen = d->exact_lengths;
  p.emax = d->exact_max_blocks;
  p.enb = d->exact_num_blocks;
  p.kc = d->k_codes;
  p.vc = d->v_codes;
  p.ks = d->k_scales;
  p.vs = d->v_scales;
  p.qtab = d->quant_table;
  p.qlen = d->quant_lengths;
  p.qmax = d->quant_max_blocks;
  p.qnb = d->quant_num_blocks;
  p.rot = d->rotation;
  dim3 grid(kBlock / 2 + 2, d->Hkv, 2 * d->B);
  const int W = code_width(d->code_bits);
  if (d->d == 64)
    launch_append_w<64>(W, grid, stream, p);
  else
    launch_append_w<128>(W, grid, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(step_commit_kernel, dim3((d->B + 63) / 64), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace akv
