// Parameter block passed by value from the host entry points to the
// attention kernels (split, chunk and merge).
#pragma once
#include <stdint.h>

namespace akv {

struct AttnParams {
  int B, Hq, Hkv, G, Tq;
  float qscale2;            // softmax scale * log2(e)
  const uint16_t* q;        // bf16 [B][Tq][Hq][d]
  const uint16_t* ek;       // exact tier pools and paging
  const uint16_t* ev;
  const int32_t* etab;
  const int32_t* elen;
  int emax, enb;
  const uint8_t* kc;        // compressed tier pools and paging
  const uint8_t* vc;
  const uint16_t* ks;
  const uint16_t* vs;
  const int32_t* qtab;
  const int32_t* qlen;
  int qmax, qnb;
  int Pe, Pq, Se, Sq;       // split tokens and splits per tier
  float* part_o;            // [B][Hkv][Sq+Se][Tq][G][d], compressed splits first
  float* part_lse;          // [B][Hkv][Sq+Se][Tq][G]
  float* o;                 // [B][Tq][Hq][d]
  float* lse;               // [B][Tq][Hq]
  // Decode split kernel only.  Workgroup (x, y, z) attends split x of
  // sequence b0 + z and writes partial row part_base + x of part_stride per
  // head.  qlen_fixed >= 0 replaces every compressed length, and qtab ==
  // nullptr means block i of a sequence's compressed tier is pool block i
  // (both for a compressed chunk streamed into a staging buffer).
  int b0, part_base, part_stride, qlen_fixed;
  // Distance between consecutive compressed-tier pool blocks: code bytes
  // (both code pools) and scale elements (both scale pools).  Separate pools
  // use Hkv*32*d and Hkv*2*d; per-block records (codes, codes, scales,
  // scales of one block together) use the record size for all four.
  size_t q_code_stride, q_scale_stride;
  // Rotation of the compressed tier: nullptr = the normalized Walsh-Hadamard
  // rotation; else a float32 [d][d] orthogonal matrix R (codes hold R x).
  // qrot: [B][Hq][d] float32 workspace for the queries rotated by R.
  const float* rot;
  int qw;  // compressed-tier code width (2, 3 or 4)
  // The call has no compressed tier: the split kernel is the exact-only one,
  // with non-temporal exact-tier V loads (every workgroup streams bf16
  // blocks; measured faster there, and slower beside compressed-tier
  // workgroups).
  int exact_nt;
  float* qrot;
  // Decode split kernel: nonzero = the workgroup in column x of unit u
  // (= y + Hkv z) takes split (x - u) mod (Sq + Se) (set for batches of
  // sequences with an even split count, so that units start on different
  // XCDs); 0 = split x.
  int split_rotate;
};

}  // namespace akv
