// Host side of the akv C ABI: argument validation (fixed order NULL -> SHAPE
// -> UNSUPPORTED -> ALIGN -> WORKSPACE, all before anything is enqueued, so a
// refused request leaves the stream untouched -- ActiveKV, "Context beyond
// VRAM", "What I built": requests that cannot be served are refused), the
// fixed split rule, workspace layout and kernel launches on the caller's
// stream.  No allocation, no synchronization, no retained pointers.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "akv_common.h"
#include "akv_params.h"

namespace akv {
hipError_t launch_decode(const AttnParams& p, int D, hipStream_t stream);
hipError_t launch_decode_splits(const AttnParams& p, int D, int splits, int seqs, hipStream_t stream);
hipError_t launch_decode_merge(const AttnParams& p, int D, hipStream_t stream);
hipError_t launch_decode_qrot(const AttnParams& p, int D, hipStream_t stream);
hipError_t launch_chunk(const AttnParams& p, int D, hipStream_t stream);
hipError_t launch_lse_merge(const float* op, const float* lp, int P, int R, int d, float* o, float* lse,
                            hipStream_t stream);
hipError_t launch_compress(const akv_compress_desc* d, hipStream_t stream);
hipError_t launch_append_evict(const akv_append_desc* d, hipStream_t stream);
hipError_t launch_ctx_save(const akv_context_desc* d, void* image, hipStream_t stream);
hipError_t launch_ctx_restore(const akv_context_desc* d, const void* image, hipStream_t stream);
void ctx_layout(const akv_context_desc* d, size_t* lens_off, size_t* exact_off, size_t* quant_off, size_t* eslot,
                size_t* qslot, size_t* total);
}  // namespace akv



namespace {

thread_local std::string g_err;

akv_status fail(akv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool width_ok(int code_bits) { return code_bits == 0 || code_bits == 2 || code_bits == 3 || code_bits == 4; }

int split_tokens(int v, int dflt) { return v ? v : dflt; }

struct Plan {
  int G, Pe, Pq, Se, Sq;  // workgroup split sizes and counts per tier (what the kernels run)
  int part_q, part_e;     // the caller-facing split (partition) sizes
  int sub;                // workgroups per partition (Pq = part_q / sub, Pe = part_e / sub)
  size_t part_rows;  // partial rows = B * Hkv * (Sq+Se) * Tq * G
  size_t qrot_off;   // rotated queries (given rotation only), after the partials
  size_t ws_bytes;
};

// Validate an attention descriptor; on success fill the plan.  staged: the
// compressed tier's pools and table live elsewhere (only its lengths and
// max_blocks are used).
akv_status check_attn(const akv_attn_desc* d, bool chunk, Plan* plan, bool staged = false) {
  // ---- NULL
  if (!d) return fail(AKV_ERR_NULL, "descriptor is NULL");
  if (d->struct_size < sizeof(akv_attn_desc))
    return fail(AKV_ERR_SHAPE, "struct_size %u < %zu", d->struct_size, sizeof(akv_attn_desc));
  if (!d->q || !d->o || !d->lse) return fail(AKV_ERR_NULL, "q, o or lse is NULL");
  const akv_exact_tier& e = d->exact;
  const akv_quant_tier& q = d->quant;
  if (e.max_blocks > 0 && (!e.k || !e.v || !e.block_table || !e.lengths))
    return fail(AKV_ERR_NULL, "exact tier present but a pointer is NULL");
  if (q.max_blocks > 0 && !q.lengths) return fail(AKV_ERR_NULL, "compressed tier present but lengths is NULL");
  if (!staged && q.max_blocks > 0 && (!q.k_codes || !q.v_codes || !q.k_scales || !q.v_scales || !q.block_table))
    return fail(AKV_ERR_NULL, "compressed tier present but a pointer is NULL");
  // ---- SHAPE
  if (d->B < 1 || d->Hq < 1 || d->Hkv < 1 || d->d < 1 || d->Tq < 1)
    return fail(AKV_ERR_SHAPE, "B, Hq, Hkv, d and Tq must be >= 1");
  if (d->Hq % d->Hkv) return fail(AKV_ERR_SHAPE, "Hq (%d) is not a multiple of Hkv (%d)", d->Hq, d->Hkv);
  if (e.max_blocks < 0 || q.max_blocks < 0) return fail(AKV_ERR_SHAPE, "max_blocks < 0");
  if ((e.max_blocks > 0 && e.num_blocks < 1) || (!staged && q.max_blocks > 0 && q.num_blocks < 1))
    return fail(AKV_ERR_SHAPE, "a present tier needs num_blocks >= 1");
  if (e.max_blocks == 0 && q.max_blocks == 0) return fail(AKV_ERR_SHAPE, "both tiers are absent");
  if (!(d->softmax_scale >= 0.0f) || !std::isfinite(d->softmax_scale))
    return fail(AKV_ERR_SHAPE, "softmax_scale must be finite and >= 0");
  if (d->split_tokens_exact < 0 || d->split_tokens_quant < 0 || d->split_tokens_exact % AKV_BLOCK_TOKENS ||
      d->split_tokens_quant % AKV_BLOCK_TOKENS)
    return fail(AKV_ERR_SHAPE, "split sizes must be non-negative multiples of %d", AKV_BLOCK_TOKENS);
  // ---- UNSUPPORTED
  if (d->d != 64 && d->d != 128) return fail(AKV_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d->d);
  const int G = d->Hq / d->Hkv;
  if (G > akv::kMaxG) return fail(AKV_ERR_UNSUPPORTED, "%d query heads per kv head (max %d)", G, akv::kMaxG);
  if (!chunk && d->Tq != 1) return fail(AKV_ERR_UNSUPPORTED, "decode takes Tq = 1 (got %d)", d->Tq);
  if (chunk && d->Tq > AKV_MAX_CHUNK) return fail(AKV_ERR_UNSUPPORTED, "chunk Tq %d > %d", d->Tq, AKV_MAX_CHUNK);
  if (chunk && e.max_blocks == 0) return fail(AKV_ERR_UNSUPPORTED, "chunk needs the exact tier (it holds the chunk)");
  if (!width_ok(d->code_bits)) return fail(AKV_ERR_UNSUPPORTED, "code_bits %d (supported: 2, 3, 4)", d->code_bits);
  if (d->B > 65535 || d->Hkv > 65535) return fail(AKV_ERR_UNSUPPORTED, "B and Hkv must be <= 65535");
  int Pe, Pq;
  if (!chunk) {
    // about AKV_DECODE_TARGET_WORKGROUPS / (B * Hkv) splits per kv head (one
    // round of workgroups): the compressed tier in the smallest multiple of
    // 256 tokens that leaves room for the exact tier at the default size, the
    // exact tier in equal runs of whole blocks over the slots left (a
    // shape-only rule, like the chunk one below)
    const long long units = (long long)d->B * d->Hkv;
    const long long budget = std::max(1LL, AKV_DECODE_TARGET_WORKGROUPS / units);
    const long long nq = (long long)q.max_blocks * AKV_BLOCK_TOKENS;
    const long long ne = (long long)e.max_blocks * AKV_BLOCK_TOKENS;
    const long long se_max = (ne + AKV_SPLIT_TOKENS_EXACT_DEFAULT - 1) / AKV_SPLIT_TOKENS_EXACT_DEFAULT;
    int pq = 0;
    for (int c = AKV_MIN_SPLIT_TOKENS; c < AKV_SPLIT_TOKENS_QUANT_DEFAULT; c += 4 * AKV_BLOCK_TOKENS)
      if ((nq + c - 1) / c + se_max <= budget) {
        pq = c;
        break;
      }
    if (pq == 0) {
      // no single round: compressed splits sized for about
      // AKV_DECODE_MANY_WORKGROUPS workgroups (a few rounds), so that every
      // workgroup's start-up is spread over more blocks; never below the default
      const long long want = (nq * units + AKV_DECODE_MANY_WORKGROUPS - 1) / AKV_DECODE_MANY_WORKGROUPS;
      const long long step = 4 * AKV_BLOCK_TOKENS;
      pq = (int)std::min<long long>(AKV_MAX_SPLIT_TOKENS,
                                    std::max<long long>(AKV_SPLIT_TOKENS_QUANT_DEFAULT, (want + step - 1) / step * step));
    }
    Pq = split_tokens(d->split_tokens_quant, pq);
    const long long rem = budget - (nq + Pq - 1) / Pq;
    int pe = AKV_SPLIT_TOKENS_EXACT_DEFAULT;
    if (rem >= 1) {
      const long long blocks = (e.max_blocks + rem - 1) / rem;
      pe = (int)std::min<long long>(AKV_SPLIT_TOKENS_EXACT_DEFAULT,
                                    std::max<long long>(AKV_MIN_SPLIT_TOKENS, blocks * AKV_BLOCK_TOKENS));
    }
    Pe = split_tokens(d->split_tokens_exact, pe);
  } else {
    // each tier in about AKV_CHUNK_TARGET_WORKGROUPS / (B * Hkv * row groups)
    // equal runs of whole blocks (a shape-only rule, like the decode one)
    const long long nrg = ((long long)d->Tq * G + AKV_CHUNK_ROWS - 1) / AKV_CHUNK_ROWS;
    const long long units = (long long)d->B * d->Hkv * nrg;
    const long long want = std::max(1LL, (AKV_CHUNK_TARGET_WORKGROUPS + units - 1) / units);
    auto dflt = [&](int max_blocks) {
      const long long blocks = std::max(1LL, (max_blocks + want - 1) / want);
      return (int)std::min<long long>(blocks * AKV_BLOCK_TOKENS, AKV_MAX_SPLIT_TOKENS);
    };
    Pe = split_tokens(d->split_tokens_exact, dflt(e.max_blocks));
    Pq = split_tokens(d->split_tokens_quant, dflt(q.max_blocks));
  }
  if (Pe > AKV_MAX_SPLIT_TOKENS || Pq > AKV_MAX_SPLIT_TOKENS)
    return fail(AKV_ERR_UNSUPPORTED, "split size above %d tokens", AKV_MAX_SPLIT_TOKENS);
  const int part_q = Pq, part_e = Pe;
  // decode grids with fewer workgroups than compute units: each split is
  // attended by `sub` workgroups of equal runs of whole blocks (a compute
  // unit streams at most ~40 GB/s, so a partition must span several), and
  // the merge takes their partials in ascending token order
  int sub = 1;
  if (!chunk) {
    const long long units = (long long)d->B * d->Hkv;
    const long long wgs = units * (((long long)q.max_blocks * AKV_BLOCK_TOKENS + Pq - 1) / Pq +
                                   ((long long)e.max_blocks * AKV_BLOCK_TOKENS + Pe - 1) / Pe);
    for (int c = AKV_DECODE_MAX_SUBSPLITS; c > 1; c >>= 1) {
      const bool fits = wgs * c <= AKV_DECODE_TARGET_WORKGROUPS / 2 &&
                        (q.max_blocks == 0 || (Pq / AKV_BLOCK_TOKENS) % (c * AKV_MIN_SUBSPLIT_BLOCKS) == 0) &&
                        (e.max_blocks == 0 || (Pe / AKV_BLOCK_TOKENS) % (c * AKV_MIN_SUBSPLIT_BLOCKS) == 0);
      if (fits) {
        sub = c;
        break;
      }
    }
    Pq /= sub;
    Pe /= sub;
  }
  const long long Se = ((long long)e.max_blocks * AKV_BLOCK_TOKENS + Pe - 1) / Pe;
  const long long Sq = ((long long)q.max_blocks * AKV_BLOCK_TOKENS + Pq - 1) / Pq;
  if (Se + Sq > AKV_MAX_SPLITS)
    return fail(AKV_ERR_UNSUPPORTED, "%lld splits per sequence (max %d): use larger splits", Se + Sq,
                AKV_MAX_SPLITS);
  if ((long long)d->Tq * d->Hq > (1LL << 30)) return fail(AKV_ERR_UNSUPPORTED, "Tq * Hq too large");
  {
    // the partials' workspace, B * Hkv * splits * Tq * G rows of d + 1 floats,
    // must stay far below the size_t range
    const double rows = (double)d->B * d->Hkv * (double)(Se + Sq) * d->Tq * G;
    if (rows * (d->d + 1) * 4.0 > (double)(1ULL << 50))
      return fail(AKV_ERR_UNSUPPORTED, "%.3g partial rows need more than 2^50 workspace bytes", rows);
  }
  // ---- ALIGN
  if (!aligned(d->q, 16)) return fail(AKV_ERR_ALIGN, "q must be 16-byte aligned");
  if (!aligned(d->rotation, 16)) return fail(AKV_ERR_ALIGN, "rotation must be 16-byte aligned");
  if (!aligned(d->o, 4) || !aligned(d->lse, 4)) return fail(AKV_ERR_ALIGN, "o and lse must be 4-byte aligned");
  if (e.max_blocks > 0 && (!aligned(e.k, 16) || !aligned(e.v, 16) || !aligned(e.block_table, 4) ||
                           !aligned(e.lengths, 4)))
    return fail(AKV_ERR_ALIGN, "exact pools must be 16-byte aligned, tables 4-byte");
  if (q.max_blocks > 0 && (!aligned(q.k_codes, 16) || !aligned(q.v_codes, 16) || !aligned(q.k_scales, 16) ||
                           !aligned(q.v_scales, 16) || !aligned(q.block_table, 4) || !aligned(q.lengths, 4)))
    return fail(AKV_ERR_ALIGN, "compressed pools must be 16-byte aligned, tables 4-byte");
  plan->G = G;
  plan->Pe = Pe;
  plan->Pq = Pq;
  plan->part_q = part_q;
  plan->part_e = part_e;
  plan->sub = sub;
  plan->Se = (int)Se;
  plan->Sq = (int)Sq;
  plan->part_rows = (size_t)d->B * d->Hkv * (size_t)(Se + Sq) * d->Tq * G;
  size_t po = plan->part_rows * d->d * sizeof(float);
  po = (po + 255) & ~(size_t)255;
  plan->ws_bytes = po + plan->part_rows * sizeof(float);
  plan->qrot_off = (plan->ws_bytes + 255) & ~(size_t)255;
  if (d->rotation) plan->ws_bytes = plan->qrot_off + (size_t)d->B * d->Tq * d->Hq * d->d * sizeof(float);
  return AKV_OK;
}

akv_status check_ws(const Plan& plan, void* ws, size_t ws_bytes) {
  if (!ws) return fail(AKV_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", plan.ws_bytes);
  if (!aligned(ws, 256)) return fail(AKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < plan.ws_bytes)
    return fail(AKV_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, plan.ws_bytes);
  return AKV_OK;
}

akv::AttnParams make_params(const akv_attn_desc* d, const Plan& plan, void* ws) {
  akv::AttnParams p{};
  p.B = d->B;
  p.Hq = d->Hq;
  p.Hkv = d->Hkv;
  p.G = plan.G;
  p.Tq = d->Tq;
  float scale = d->softmax_scale > 0.0f ? d->softmax_scale : 1.0f / std::sqrt((float)d->d);
  p.qscale2 = scale * akv::kLog2e;
  p.q = d->q;
  p.ek = d->exact.k;
  p.ev = d->exact.v;
  p.etab = d->exact.block_table;
  p.elen = d->exact.lengths;
  p.emax = d->exact.max_blocks;
  p.enb = d->exact.num_blocks;
  p.kc = d->quant.k_codes;
  p.vc = d->quant.v_codes;
  p.ks = d->quant.k_scales;
  p.vs = d->quant.v_scales;
  p.qtab = d->quant.block_table;
  p.qlen = d->quant.lengths;
  p.qmax = d->quant.max_blocks;
  p.qnb = d->quant.num_blocks;
  p.Pe = plan.Pe;
  p.Pq = plan.Pq;
  p.Se = plan.Se;
  p.Sq = plan.Sq;
  size_t po = plan.part_rows * d->d * sizeof(float);
  po = (po + 255) & ~(size_t)255;
  char* base = static_cast<char*>(ws);
  p.part_o = reinterpret_cast<float*>(base);
  p.part_lse = reinterpret_cast<float*>(base + po);
  p.o = d->o;
  p.lse = d->lse;
  p.b0 = 0;
  p.part_base = 0;
  p.part_stride = plan.Sq + plan.Se;
  p.qlen_fixed = -1;
  p.qw = akv::code_width(d->code_bits);
  p.exact_nt = d->quant.max_blocks == 0;
  p.q_code_stride = (size_t)d->Hkv * 8 * p.qw * d->d;
  p.q_scale_stride = (size_t)d->Hkv * 2 * d->d;
  p.rot = d->rotation;
  p.qrot = d->rotation ? reinterpret_cast<float*>(base + plan.qrot_off) : nullptr;
  return p;
}

akv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return AKV_OK;
  return fail(AKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int akv_abi_version(void) { return AKV_ABI_VERSION; }

const char* akv_last_error(void) { return g_err.c_str(); }

size_t akv_decode_workspace_bytes(const akv_attn_desc* desc) {
  Plan plan;
  return check_attn(desc, false, &plan) == AKV_OK ? plan.ws_bytes : 0;
}

int32_t akv_decode_split_workgroups(const akv_attn_desc* desc) {
  Plan plan;
  return check_attn(desc, false, &plan) == AKV_OK ? plan.sub : 0;
}

size_t akv_chunk_workspace_bytes(const akv_attn_desc* desc) {
  Plan plan;
  return check_attn(desc, true, &plan) == AKV_OK ? plan.ws_bytes : 0;
}

akv_status akv_split_plan(const akv_attn_desc* desc, int32_t chunk, int32_t* out) {
  Plan plan;
  akv_status s = check_attn(desc, chunk != 0, &plan);
  if (s != AKV_OK) return s;
  if (!out) return fail(AKV_ERR_NULL, "out is NULL");
  out[0] = plan.part_q;
  out[1] = plan.part_e;
  out[2] = (plan.Sq + plan.sub - 1) / plan.sub;
  out[3] = (plan.Se + plan.sub - 1) / plan.sub;
  return AKV_OK;
}

akv_status akv_attend_decode(const akv_attn_desc* desc, void* ws, size_t ws_bytes, void* stream) {
  Plan plan;
  akv_status s = check_attn(desc, false, &plan);
  if (s != AKV_OK) return s;
  if ((s = check_ws(plan, ws, ws_bytes)) != AKV_OK) return s;
  akv::AttnParams p = make_params(desc, plan, ws);
  return hip_status(akv::launch_decode(p, desc->d, static_cast<hipStream_t>(stream)), "akv_attend_decode");
}

}  // extern "C"

// ------------------------------------------------ allocation-free decode
// The library's own scratch for akv_attend_decode_noalloc: one array per GPU,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory, so the kernels only ever get the device
// address that hipGetSymbolAddress returns for the current GPU.
static __device__ __align__(256) unsigned char scratch[AKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per GPU, once looked up

// The current GPU's scratch address, looked up on its first call there.
akv_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(AKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(AKV_ERR_UNSUPPORTED, "device %d (at most %d served)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(AKV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return AKV_OK;
}

}  // namespace

extern "C" {

akv_status akv_attend_decode_noalloc(const akv_attn_desc* desc, void* stream) {
  Plan plan;
  akv_status s = check_attn(desc, false, &plan);
  if (s != AKV_OK) return s;
  if (plan.ws_bytes > AKV_NOALLOC_SCRATCH_BYTES)
    return fail(AKV_ERR_WORKSPACE, "this shape needs %zu bytes of scratch; the library's own holds %zu "
                "(use akv_attend_decode with a workspace)", plan.ws_bytes, (size_t)AKV_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((s = scratch_for_current_device(&ws)) != AKV_OK) return s;
  akv::AttnParams p = make_params(desc, plan, ws);
  return hip_status(akv::launch_decode(p, desc->d, static_cast<hipStream_t>(stream)), "akv_attend_decode_noalloc");
}

// Validation of the staging descriptor, one category at a time (the caller
// interleaves the categories with the attention descriptor's).
akv_status check_staging(const akv_attn_desc* desc, const akv_staging_desc* st, akv_status category) {
  if (category == AKV_ERR_NULL) {
    if (!st) return fail(AKV_ERR_NULL, "staging descriptor is NULL");
    if (st->struct_size >= sizeof(akv_staging_desc)) {
      if (!st->seqs || !st->ring || !st->copy_stream || !st->events)
        return fail(AKV_ERR_NULL, "a staging pointer is NULL");
      for (int i = 0; i < 2 * st->slots + 1 && st->slots >= 2; ++i)
        if (!st->events[i]) return fail(AKV_ERR_NULL, "staging event %d is NULL", i);
      const int nb = (desc && desc->struct_size >= sizeof(akv_attn_desc) && desc->B <= 65535) ? desc->B : 0;
      for (int b = 0; b < nb; ++b) {
        const akv_host_tier& h = st->seqs[b];
        if (h.length > 0 && !h.blocks) return fail(AKV_ERR_NULL, "host tier %d: blocks is NULL", b);
      }
    }
  } else if (category == AKV_ERR_SHAPE) {
    if (st->struct_size < sizeof(akv_staging_desc))
      return fail(AKV_ERR_SHAPE, "staging struct_size %u < %zu", st->struct_size, sizeof(akv_staging_desc));
    if (st->slots < 2) return fail(AKV_ERR_SHAPE, "staging needs >= 2 slots");
    const long long cap = (long long)desc->quant.max_blocks * AKV_BLOCK_TOKENS;
    for (int b = 0; b < desc->B; ++b)
      if (st->seqs[b].length < 0 || st->seqs[b].length > cap)
        return fail(AKV_ERR_SHAPE, "host tier %d: length %d outside [0, %lld]", b, st->seqs[b].length, cap);
  } else if (category == AKV_ERR_ALIGN) {
    if (!aligned(st->ring, 256)) return fail(AKV_ERR_ALIGN, "staging ring must be 256-byte aligned");
    for (int b = 0; b < desc->B; ++b) {
      const akv_host_tier& h = st->seqs[b];
      if (h.length > 0 && !aligned(h.blocks, 16))
        return fail(AKV_ERR_ALIGN, "host tier %d: blocks must be 16-byte aligned", b);
    }
  }
  return AKV_OK;
}

// Position of a status in the validation order NULL -> SHAPE -> UNSUPPORTED -> ALIGN -> WORKSPACE.
int status_rank(akv_status s) {
  switch (s) {
    case AKV_ERR_NULL: return 0;
    case AKV_ERR_SHAPE: return 1;
    case AKV_ERR_UNSUPPORTED: return 2;
    case AKV_ERR_ALIGN: return 3;
    case AKV_ERR_WORKSPACE: return 4;
    default: return 5;
  }
}

akv_status akv_attend_decode_staged(const akv_attn_desc* desc, const akv_staging_desc* st, void* ws,
                                    size_t ws_bytes, void* stream) {
  Plan plan;
  // NULL of both descriptors first, then the remaining categories in order
  akv_status s = check_staging(desc, st, AKV_ERR_NULL);
  if (s != AKV_OK) {
    if (!desc) return fail(AKV_ERR_NULL, "descriptor is NULL");
    return s;
  }
  akv_status sa = check_attn(desc, false, &plan, true);
  if (sa == AKV_ERR_NULL) return sa;
  const std::string attn_msg = g_err;
  for (akv_status c : {AKV_ERR_SHAPE, AKV_ERR_UNSUPPORTED, AKV_ERR_ALIGN}) {
    if (sa != AKV_OK && status_rank(sa) <= status_rank(c)) {
      g_err = attn_msg;
      return sa;
    }
    if ((s = check_staging(desc, st, c)) != AKV_OK) return s;
  }
  if (sa != AKV_OK) {
    g_err = attn_msg;
    return sa;
  }
  if ((s = check_ws(plan, ws, ws_bytes)) != AKV_OK) return s;
  const akv_quant_tier& q = desc->quant;
  // ring slots of whole compressed splits; a block is one record of
  // Hkv*8*w*d K-code, Hkv*8*w*d V-code (code width w), Hkv*2*d K-scale and
  // Hkv*2*d V-scale bytes / halves
  const int D = desc->d, H = desc->Hkv;
  const size_t code_bytes = (size_t)H * 8 * akv::code_width(desc->code_bits) * D, scale_bytes = (size_t)H * 4 * D;
  const size_t block_bytes = 2 * code_bytes + 2 * scale_bytes;
  const size_t slot_bytes = (st->ring_bytes / st->slots) & ~(size_t)255;
  const int slot_blocks = (int)std::min<size_t>(slot_bytes / block_bytes, 1 << 30);
  const int split_blocks = plan.Pq / AKV_BLOCK_TOKENS;
  const int chunk_splits = slot_blocks / split_blocks;
  if (q.max_blocks > 0 && chunk_splits < 1)
    return fail(AKV_ERR_WORKSPACE, "staging slots of %zu bytes hold %d blocks; one split needs %d", slot_bytes,
                slot_blocks, split_blocks);
  hipStream_t cs = static_cast<hipStream_t>(stream), xs = static_cast<hipStream_t>(st->copy_stream);
  hipEvent_t* ev = reinterpret_cast<hipEvent_t*>(const_cast<void**>(st->events));
  const akv::AttnParams base = make_params(desc, plan, ws);
  hipError_t e;
#define AKV_HIP(call)                                          \
  do {                                                         \
    if ((e = (call)) != hipSuccess) return hip_status(e, #call); \
  } while (0)
  // slots may still be read by work already on `stream` (an earlier call)
  AKV_HIP(hipEventRecord(ev[2 * st->slots], cs));
  AKV_HIP(hipStreamWaitEvent(xs, ev[2 * st->slots], 0));
  // queries rotated by a given rotation, then the exact-tier splits of every
  // sequence (they overlap the first copies)
  AKV_HIP(akv::launch_decode_qrot(base, D, cs));
  if (plan.Se > 0) {
    akv::AttnParams p = base;
    p.Sq = 0;
    p.part_base = plan.Sq;
    AKV_HIP(akv::launch_decode_splits(p, D, plan.Se, desc->B, cs));
  }
  // compressed chunks through the ring, one copy each
  long long k = 0;
  for (int b = 0; b < desc->B; ++b) {
    const akv_host_tier& h = st->seqs[b];
    const int ns = (h.length + plan.Pq - 1) / plan.Pq;
    for (int s0 = 0; s0 < ns; s0 += chunk_splits) {
      const int n = std::min(chunk_splits, ns - s0);
      const int tok0 = s0 * plan.Pq, ntok = std::min(h.length - tok0, n * plan.Pq);
      const int blk0 = tok0 / AKV_BLOCK_TOKENS, nblk = (ntok + AKV_BLOCK_TOKENS - 1) / AKV_BLOCK_TOKENS;
      const int slot = (int)(k % st->slots);
      unsigned char* sb = static_cast<unsigned char*>(st->ring) + (size_t)slot * slot_bytes;
      if (k >= st->slots) AKV_HIP(hipStreamWaitEvent(xs, ev[st->slots + slot], 0));  // slot free
      AKV_HIP(hipMemcpyAsync(sb, static_cast<const unsigned char*>(h.blocks) + (size_t)blk0 * block_bytes,
                             (size_t)nblk * block_bytes, hipMemcpyHostToDevice, xs));
      AKV_HIP(hipEventRecord(ev[slot], xs));  // slot ready
      AKV_HIP(hipStreamWaitEvent(cs, ev[slot], 0));
      akv::AttnParams p = base;
      p.b0 = b;
      p.Sq = n;
      p.Se = 0;
      p.part_base = s0;
      p.kc = sb;
      p.vc = sb + code_bytes;
      p.ks = reinterpret_cast<const uint16_t*>(sb + 2 * code_bytes);
      p.vs = reinterpret_cast<const uint16_t*>(sb + 2 * code_bytes + scale_bytes);
      p.q_code_stride = block_bytes;
      p.q_scale_stride = block_bytes / 2;
      p.qtab = nullptr;
      p.qlen_fixed = ntok;
      p.qmax = slot_blocks;
      p.qnb = slot_blocks;
      AKV_HIP(akv::launch_decode_splits(p, D, n, 1, cs));
      AKV_HIP(hipEventRecord(ev[st->slots + slot], cs));  // slot free once this kernel is done
      ++k;
    }
  }
  AKV_HIP(akv::launch_decode_merge(base, D, cs));
#undef AKV_HIP
  return AKV_OK;
}

akv_status akv_attend_chunk(const akv_attn_desc* desc, void* ws, size_t ws_bytes, void* stream) {
  Plan plan;
  akv_status s = check_attn(desc, true, &plan);
  if (s != AKV_OK) return s;
  if ((s = check_ws(plan, ws, ws_bytes)) != AKV_OK) return s;
  akv::AttnParams p = make_params(desc, plan, ws);
  return hip_status(akv::launch_chunk(p, desc->d, static_cast<hipStream_t>(stream)), "akv_attend_chunk");
}

akv_status akv_lse_merge(const float* o_parts, const float* lse_parts, int32_t P, int32_t R, int32_t d,
                         float* o_out, float* lse_out, void* stream) {
  if (!o_parts || !lse_parts || !o_out || !lse_out) return fail(AKV_ERR_NULL, "a merge pointer is NULL");
  if (P < 1 || R < 0 || d < 1) return fail(AKV_ERR_SHAPE, "need P >= 1, R >= 0, d >= 1");
  if (P > 4096 || d > 1024) return fail(AKV_ERR_UNSUPPORTED, "P <= 4096 and d <= 1024 are served");
  if (!aligned(o_parts, 4) || !aligned(lse_parts, 4) || !aligned(o_out, 4) || !aligned(lse_out, 4))
    return fail(AKV_ERR_ALIGN, "merge buffers must be 4-byte aligned");
  if (R == 0) return AKV_OK;
  return hip_status(akv::launch_lse_merge(o_parts, lse_parts, P, R, d, o_out, lse_out,
                                          static_cast<hipStream_t>(stream)),
                    "akv_lse_merge");
}

akv_status akv_compress_evicted(const akv_compress_desc* d, void* stream) {
  if (!d) return fail(AKV_ERR_NULL, "descriptor is NULL");
  if (d->struct_size < sizeof(akv_compress_desc))
    return fail(AKV_ERR_SHAPE, "struct_size %u < %zu", d->struct_size, sizeof(akv_compress_desc));
  if (!d->src_k || !d->src_v || !d->src_block_table || !d->dst_k_codes || !d->dst_v_codes || !d->dst_k_scales ||
      !d->dst_v_scales || !d->dst_block_table)
    return fail(AKV_ERR_NULL, "a compress pointer is NULL");
  if (d->Hkv < 1 || d->d < 1 || d->n_tokens < 0 || d->src_start < 0 || d->dst_start < 0 || d->src_max_blocks < 1 ||
      d->dst_max_blocks < 1 || d->src_num_blocks < 1 || d->dst_num_blocks < 1)
    return fail(AKV_ERR_SHAPE, "compress sizes out of range");
  if ((long long)d->src_start + d->n_tokens > (long long)d->src_max_blocks * AKV_BLOCK_TOKENS ||
      (long long)d->dst_start + d->n_tokens > (long long)d->dst_max_blocks * AKV_BLOCK_TOKENS)
    return fail(AKV_ERR_SHAPE, "token range exceeds a block table");
  if (d->d != 64 && d->d != 128) return fail(AKV_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d->d);
  if (!width_ok(d->code_bits)) return fail(AKV_ERR_UNSUPPORTED, "code_bits %d (supported: 2, 3, 4)", d->code_bits);
  if (d->Hkv > 65535) return fail(AKV_ERR_UNSUPPORTED, "Hkv must be <= 65535");
  if (!aligned(d->src_k, 2) || !aligned(d->src_v, 2) || !aligned(d->dst_k_scales, 2) ||
      !aligned(d->dst_v_scales, 2) || !aligned(d->src_block_table, 4) || !aligned(d->dst_block_table, 4))
    return fail(AKV_ERR_ALIGN, "compress buffers misaligned");
  if (!aligned(d->rotation, 16)) return fail(AKV_ERR_ALIGN, "rotation must be 16-byte aligned");
  if (d->n_tokens == 0) return AKV_OK;
  return hip_status(akv::launch_compress(d, static_cast<hipStream_t>(stream)), "akv_compress_evicted");
}

akv_status akv_append_evict(const akv_append_desc* d, void* stream) {
  if (!d) return fail(AKV_ERR_NULL, "descriptor is NULL");
  if (d->struct_size < sizeof(akv_append_desc))
    return fail(AKV_ERR_SHAPE, "struct_size %u < %zu", d->struct_size, sizeof(akv_append_desc));
  if (!d->new_k || !d->new_v || !d->exact_k || !d->exact_v || !d->exact_table || !d->exact_lengths ||
      !d->k_codes || !d->v_codes || !d->k_scales || !d->v_scales || !d->quant_table || !d->quant_lengths)
    return fail(AKV_ERR_NULL, "an append pointer is NULL");
  if (d->B < 1 || d->Hkv < 1 || d->d < 1 || d->exact_max_blocks < 1 || d->exact_num_blocks < 1 ||
      d->quant_max_blocks < 1 || d->quant_num_blocks < 1)
    return fail(AKV_ERR_SHAPE, "append sizes out of range");
  if (d->window < AKV_BLOCK_TOKENS || d->window % AKV_BLOCK_TOKENS)
    return fail(AKV_ERR_SHAPE, "window %d must be a positive multiple of %d", d->window, AKV_BLOCK_TOKENS);
  if (d->window / AKV_BLOCK_TOKENS + 1 > d->exact_max_blocks)
    return fail(AKV_ERR_SHAPE, "window %d needs %d exact-table entries (have %d)", d->window,
                d->window / AKV_BLOCK_TOKENS + 1, d->exact_max_blocks);
  if (d->d != 64 && d->d != 128) return fail(AKV_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d->d);
  if (!width_ok(d->code_bits)) return fail(AKV_ERR_UNSUPPORTED, "code_bits %d (supported: 2, 3, 4)", d->code_bits);
  if (d->B > 32767 || d->Hkv > 65535) return fail(AKV_ERR_UNSUPPORTED, "B must be <= 32767 and Hkv <= 65535");
  if (!aligned(d->new_k, 2) || !aligned(d->new_v, 2) || !aligned(d->exact_k, 2) || !aligned(d->exact_v, 2) ||
      !aligned(d->k_scales, 2) || !aligned(d->v_scales, 2) || !aligned(d->exact_table, 4) ||
      !aligned(d->exact_lengths, 4) || !aligned(d->quant_table, 4) || !aligned(d->quant_lengths, 4) ||
      !aligned(d->rotation, 16))
    return fail(AKV_ERR_ALIGN, "append buffers misaligned");
  return hip_status(akv::launch_append_evict(d, static_cast<hipStream_t>(stream)), "akv_append_evict");
}

// ---------------------------------------------------------- context checkpoint
static akv_status check_context(const akv_context_desc* d, const void* image, bool need_image, size_t* bytes) {
  if (!d) return fail(AKV_ERR_NULL, "descriptor is NULL");
  if (d->struct_size < sizeof(akv_context_desc))
    return fail(AKV_ERR_SHAPE, "struct_size %u < %zu", d->struct_size, sizeof(akv_context_desc));
  if (!d->exact_lengths || !d->quant_lengths) return fail(AKV_ERR_NULL, "a lengths pointer is NULL");
  if (d->exact_max_blocks > 0 && (!d->exact_k || !d->exact_v || !d->exact_table))
    return fail(AKV_ERR_NULL, "exact tier present but a pointer is NULL");
  if (d->quant_max_blocks > 0 && (!d->k_codes || !d->v_codes || !d->k_scales || !d->v_scales || !d->quant_table))
    return fail(AKV_ERR_NULL, "compressed tier present but a pointer is NULL");
  if (need_image && !image) return fail(AKV_ERR_NULL, "image is NULL");
  if (d->B < 1 || d->Hkv < 1 || d->d < 1 || d->exact_max_blocks < 0 || d->quant_max_blocks < 0)
    return fail(AKV_ERR_SHAPE, "context sizes out of range");
  if ((d->exact_max_blocks > 0 && d->exact_num_blocks < 1) || (d->quant_max_blocks > 0 && d->quant_num_blocks < 1))
    return fail(AKV_ERR_SHAPE, "a present tier needs num_blocks >= 1");
  if (d->d != 64 && d->d != 128) return fail(AKV_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d->d);
  if (!width_ok(d->code_bits)) return fail(AKV_ERR_UNSUPPORTED, "code_bits %d (supported: 2, 3, 4)", d->code_bits);
  if (d->B > 65535 || d->exact_max_blocks > (1 << 30) || d->quant_max_blocks > (1 << 30))
    return fail(AKV_ERR_UNSUPPORTED, "B must be <= 65535");
  if (!aligned(d->exact_k, 16) || !aligned(d->exact_v, 16) || !aligned(d->k_codes, 16) || !aligned(d->v_codes, 16) ||
      !aligned(d->k_scales, 16) || !aligned(d->v_scales, 16) || !aligned(d->exact_table, 4) ||
      !aligned(d->quant_table, 4) || !aligned(d->exact_lengths, 4) || !aligned(d->quant_lengths, 4))
    return fail(AKV_ERR_ALIGN, "pools must be 16-byte aligned, tables and lengths 4-byte");
  if (need_image && !aligned(image, 256)) return fail(AKV_ERR_ALIGN, "image must be 256-byte aligned");
  size_t lo, eo, qo, es, qs;
  akv::ctx_layout(d, &lo, &eo, &qo, &es, &qs, bytes);
  return AKV_OK;
}

size_t akv_checkpoint_bytes(const akv_context_desc* desc) {
  size_t n = 0;
  return check_context(desc, nullptr, false, &n) == AKV_OK ? n : 0;
}

akv_status akv_checkpoint_save(const akv_context_desc* desc, void* image, void* stream) {
  size_t n = 0;
  akv_status s = check_context(desc, image, true, &n);
  if (s != AKV_OK) return s;
  return hip_status(akv::launch_ctx_save(desc, image, static_cast<hipStream_t>(stream)), "akv_checkpoint_save");
}

akv_status akv_checkpoint_restore(const akv_context_desc* desc, const void* image, void* stream) {
  size_t n = 0;
  akv_status s = check_context(desc, image, true, &n);
  if (s != AKV_OK) return s;
  return hip_status(akv::launch_ctx_restore(desc, image, static_cast<hipStream_t>(stream)), "akv_checkpoint_restore");
}

}  // extern "C"
