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
};

}  // namespace akv
