// Context checkpoint: a fixed-format image of a batch's two-tier history
// (ActiveKV, "Context beyond VRAM", "What I built": a context can be parked
// and brought back later without being rebuilt from its tokens).  The image holds the
// lengths and, slot by slot in token order, the bytes of every block below
// each length; restore writes those bytes into whatever pool blocks the
// caller's tables name.  Pure data movement: one workgroup of 256 threads per
// (block slot, sequence, tier), 16-byte copies.
#include "akv_common.h"

namespace akv {

constexpr int kCtxThreads = 256;
constexpr uint32_t kCtxMagic0 = 0x43564B41u;  // "AKVC"
constexpr uint32_t kCtxMagic1 = 0x31305854u;  // "TX01"

struct CtxParams {
  int B, Hkv, d;
  uint16_t* ek;
  uint16_t* ev;
  const int32_t* etab;
  int32_t* elen;
  int emax, enb;
  uint8_t* kc;
  uint8_t* vc;
  uint16_t* ks;
  uint16_t* vs;
  const int32_t* qtab;
  int32_t* qlen;
  int qmax, qnb;
  int qw;                                 // code width (2, 3 or 4)
  size_t lens_off, exact_off, quant_off;  // image offsets
  size_t eslot, qslot;                    // bytes per slot
};

// Byte regions of one slot, in image order: a pool region of `bytes` bytes
// per region index.
struct Region {
  unsigned char* pool;
  size_t bytes;
};

__device__ inline int slot_regions(const CtxParams& p, int tier, int pb, Region (&r)[4]) {
  const size_t H = p.Hkv, D = p.d;
  if (tier == 0) {
    const size_t n = H * kBlock * D * 2;  // Hkv slabs of 64 x d bf16
    r[0] = {reinterpret_cast<unsigned char*>(p.ek) + pb * n, n};
    r[1] = {reinterpret_cast<unsigned char*>(p.ev) + pb * n, n};
    return 2;
  }
  const size_t nc = H * 8 * p.qw * D, ns = H * 4 * D;
  r[0] = {p.kc + pb * nc, nc};
  r[1] = {p.vc + pb * nc, nc};
  r[2] = {reinterpret_cast<unsigned char*>(p.ks) + pb * ns, ns};
  r[3] = {reinterpret_cast<unsigned char*>(p.vs) + pb * ns, ns};
  return 4;
}

// Pool block of slot j of sequence b in tier t, or -1 when the slot holds no
// tokens (at or past the length) or the table entry is outside the pool.
__device__ inline int slot_block(const CtxParams& p, int tier, int b, int j, int len) {
  const int maxb = tier ? p.qmax : p.emax, nb = tier ? p.qnb : p.enb;
  if (len < 0 || len > maxb * kBlock || j >= (len + kBlock - 1) / kBlock) return -1;
  const int pb = (tier ? p.qtab : p.etab)[(size_t)b * maxb + j];
  return (pb >= 0 && pb < nb) ? pb : -1;
}

// Regions never overlap; four loads go out before their stores.
__device__ inline void copy16(unsigned char* __restrict__ dst, const unsigned char* __restrict__ src, size_t bytes) {
  constexpr size_t kStep = 16 * kCtxThreads;
  size_t i = 16 * threadIdx.x;
  for (; i + 3 * kStep < bytes; i += 4 * kStep) {
    u32x4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const u32x4*>(src + i + u * kStep);
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4*>(dst + i + u * kStep) = x[u];
  }
  for (; i < bytes; i += kStep) *reinterpret_cast<u32x4*>(dst + i) = *reinterpret_cast<const u32x4*>(src + i);
}

__device__ inline void zero16(unsigned char* dst, size_t bytes) {
  for (size_t i = 16 * threadIdx.x; i < bytes; i += 16 * kCtxThreads)
    *reinterpret_cast<u32x4*>(dst + i) = u32x4{0, 0, 0, 0};
}

// grid (max(emax, qmax), B, 2): slot j of sequence b in tier z.
__global__ __launch_bounds__(kCtxThreads) void ctx_save_kernel(CtxParams p, unsigned char* img) {
  const int j = blockIdx.x, b = blockIdx.y, tier = blockIdx.z;
  if (j == 0 && b == 0 && tier == 0) {
    // header and lengths (the rest of [0, exact_off) is zero)
    for (size_t i = 4 * threadIdx.x; i < p.exact_off; i += 4 * kCtxThreads) {
      uint32_t v = 0;
      if (i == 0) v = kCtxMagic0;
      else if (i == 4) v = kCtxMagic1;
      else if (i >= 8 && i < 32) {
        const int f = (int)(i - 8) / 4;
        v = (uint32_t)(f == 0 ? p.B : f == 1 ? p.Hkv : f == 2 ? p.d : f == 3 ? p.emax : f == 4 ? p.qmax : p.qw);
      } else if (i >= p.lens_off && i < p.lens_off + 8 * (size_t)p.B) {
        const int k = (int)(i - p.lens_off) / 4;
        v = (uint32_t)((k & 1) ? p.qlen[k >> 1] : p.elen[k >> 1]);
      }
      *reinterpret_cast<uint32_t*>(img + i) = v;
    }
  }
  const int maxb = tier ? p.qmax : p.emax;
  if (j >= maxb) return;
  const int len = tier ? p.qlen[b] : p.elen[b];
  const int pb = slot_block(p, tier, b, j, len);
  unsigned char* dst =
      img + (tier ? p.quant_off + ((size_t)b * p.qmax + j) * p.qslot : p.exact_off + ((size_t)b * p.emax + j) * p.eslot);
  Region r[4];
  const int nr = slot_regions(p, tier, pb < 0 ? 0 : pb, r);
  for (int k = 0; k < nr; ++k) {
    if (pb >= 0) copy16(dst, r[k].pool, r[k].bytes);
    else zero16(dst, r[k].bytes);
    dst += r[k].bytes;
  }
}

__device__ inline bool header_ok(const CtxParams& p, const unsigned char* img) {
  const uint32_t* h = reinterpret_cast<const uint32_t*>(img);
  return h[0] == kCtxMagic0 && h[1] == kCtxMagic1 && (int)h[2] == p.B && (int)h[3] == p.Hkv && (int)h[4] == p.d &&
         (int)h[5] == p.emax && (int)h[6] == p.qmax && (int)h[7] == p.qw;
}

__global__ __launch_bounds__(kCtxThreads) void ctx_restore_kernel(CtxParams p, const unsigned char* img) {
  const int j = blockIdx.x, b = blockIdx.y, tier = blockIdx.z;
  const bool hok = header_ok(p, img);
  const int32_t* lens = reinterpret_cast<const int32_t*>(img + p.lens_off);
  if (j == 0 && tier == 0) {
    // lengths of sequence b, once every slot below them has a valid block
    const int el = hok ? lens[2 * b] : -1, ql = hok ? lens[2 * b + 1] : -1;
    const bool lok = el >= 0 && el <= p.emax * kBlock && ql >= 0 && ql <= p.qmax * kBlock;
    int bad = !lok;
    if (lok) {
      const int ne = (el + kBlock - 1) / kBlock, nq = (ql + kBlock - 1) / kBlock;
      for (int i = threadIdx.x; i < ne + nq; i += kCtxThreads) {
        const bool q = i >= ne;
        const int pb = q ? p.qtab[(size_t)b * p.qmax + (i - ne)] : p.etab[(size_t)b * p.emax + i];
        if (pb < 0 || pb >= (q ? p.qnb : p.enb)) bad = 1;
      }
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) {
      p.elen[b] = bad ? -1 : el;
      if (p.qmax) p.qlen[b] = bad ? 0 : ql;
    }
  }
  if (!hok) return;
  const int maxb = tier ? p.qmax : p.emax;
  if (j >= maxb) return;
  const int pb = slot_block(p, tier, b, j, lens[2 * b + tier]);
  if (pb < 0) return;
  const unsigned char* src =
      img + (tier ? p.quant_off + ((size_t)b * p.qmax + j) * p.qslot : p.exact_off + ((size_t)b * p.emax + j) * p.eslot);
  Region r[4];
  const int nr = slot_regions(p, tier, pb, r);
  for (int k = 0; k < nr; ++k) {
    copy16(r[k].pool, src, r[k].bytes);
    src += r[k].bytes;
  }
}

// Image layout sizes for a shape (shared by the byte count and the kernels).
void ctx_layout(const akv_context_desc* d, size_t* lens_off, size_t* exact_off, size_t* quant_off, size_t* eslot,
                size_t* qslot, size_t* total) {
  const size_t H = d->Hkv, D = d->d, B = d->B;
  *lens_off = 256;
  *exact_off = 256 + ((8 * B + 255) / 256) * 256;
  *eslot = 256 * H * D;
  *qslot = (16 * (size_t)code_width(d->code_bits) + 8) * H * D;
  *quant_off = *exact_off + B * (size_t)d->exact_max_blocks * *eslot;
  *total = *quant_off + B * (size_t)d->quant_max_blocks * *qslot;
}

static CtxParams ctx_params(const akv_context_desc* d) {
  CtxParams p;
  p.B = d->B;
  p.Hkv = d->Hkv;
  p.d = d->d;
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
  p.qw = code_width(d->code_bits);
  size_t total;
  ctx_layout(d, &p.lens_off, &p.exact_off, &p.quant_off, &p.eslot, &p.qslot, &total);
  return p;
}

hipError_t launch_ctx_save(const akv_context_desc* d, void* image, hipStream_t stream) {
  const CtxParams p = ctx_params(d);
  dim3 grid(max(1, max(d->exact_max_blocks, d->quant_max_blocks)), d->B, 2);
  hipLaunchKernelGGL(ctx_save_kernel, grid, dim3(kCtxThreads), 0, stream, p, static_cast<unsigned char*>(image));
  return hipGetLastError();
}

hipError_t launch_ctx_restore(const akv_context_desc* d, const void* image, hipStream_t stream) {
  const CtxParams p = ctx_params(d);
  dim3 grid(max(1, max(d->exact_max_blocks, d->quant_max_blocks)), d->B, 2);
  hipLaunchKernelGGL(ctx_restore_kernel, grid, dim3(kCtxThreads), 0, stream, p,
                     static_cast<const unsigned char*>(image));
  return hipGetLastError();
}

}  // namespace akv
