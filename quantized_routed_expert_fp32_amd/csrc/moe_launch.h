// Kernel argument blocks and launchers (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct RouteArgs {
  const uint8_t* base;
  uint64_t r_off, r_soff, g_off, g_soff;
  const uint16_t* x;
  int act_fp16, H, E, k, R;
  const float* bias;
  int32_t* ids;
  float* p;
  float* sg;
  float* logits;   // tap [R, E+1] or null
  float* lg_ws;    // [R, E] scratch: logits before the bias
  float* gl_ws;    // [R] scratch: gate-row logits
  uint64_t* cand;  // [R, 32] tile picks: epoch << 40 | id << 32 | value bits
  uint32_t* sync;  // [0] epoch state, [1] completed workgroups, [2] failed rows (sticky)
  int wait_limit;  // polls of the hand-off before a row is reported as not handed off
  int sticky;      // 1: a failure count already in sync[2] marks this call's rows failed
};

// Offsets of one expert class (routed or shared) inside the packed layer.
struct ExpertClass {
  uint64_t base_off, stride;          // expert e at base_off + e*stride
  uint64_t gu_codes, gu_scales, dn_codes, dn_scales;   // inside an expert block
  uint32_t blk_bytes;                 // bytes of one expert block
  int inter;
};

struct DecodeArgs {
  const uint8_t* base;
  ExpertClass rt, sh;
  const uint16_t* x;
  int act_fp16, H, E, k, R, Imax;
  const int32_t* ids;
  const float* p;
  const float* sg;
  uint16_t* hhi;  // [R, k+1, Imax] fp16 high part of h
  uint16_t* hlo;  // [R, k+1, Imax] fp16 low part of h (h - hi)
  float* hc;      // [R, k+1, Imax/32] chunk sums of hi + lo
  float* y;       // [R, H]
  float* tap_gu;  // [R, k+1, 2, Imax] or null
  float* tap_h;   // [R, k+1, Imax] or null
  float* tap_e;   // [R, k+1, H] or null
  // the exact chunk form only (null otherwise): the sort's expert-major
  // slot order, its list of expert blocks (expert, first position, rows <=
  // 16) and the block count on the device
  const int32_t* perm;
  const int32_t* blocks;
  const int32_t* nblocks;
  float* e_ws;    // [R*(k+1), H] fp32 slot outputs (exact chunk form)
};

struct GroupedArgs {
  const uint8_t* base;
  ExpertClass rt, sh;
  const uint16_t* x;
  int act_fp16, H, E, k, R, Imax;
  const int32_t* ids;
  const float* p;
  const float* sg;
  const uint16_t* x16;  // [R, H] fp16 activations for the GEMMs (x itself, or a copy of bf16 x)
  int32_t* meta;     // tile count, queue counters, expert offsets
  int32_t* perm;     // expert-major position -> slot index r*(k+1)+j
  uint16_t* hbuf;    // [R*(k+1), Imax] fp16 bits (expert-major order)
  float* e_ws;       // [R*(k+1), H] slot order
  int32_t* tiles;    // work list of M-tiles (expert, first position, rows)
  int max_tiles;     // capacity of the list
  int blk16;         // nonzero: the list holds blocks of at most 16 rows (the exact chunk form)
  float* y;
  float* tap_gu;
  float* tap_h;
  float* tap_e;
};

// ev: NULL or 8 events; ev[2i] / ev[2i+1] (each may be NULL) bracket kernel i
hipError_t launch_route(int fr, int fg, const RouteArgs& a, hipStream_t s, hipEvent_t* ev);
hipError_t launch_decode(int fr, int fs, const DecodeArgs& a, hipStream_t s, hipEvent_t* ev);
// The exact chunk form: the sort alone (16-row blocks), the router with the
// decode router's per-row arithmetic for any number of rows, and gate/up on
// expert blocks followed by the decode down + combine over every row.
hipError_t launch_grp_sort(const GroupedArgs& a, hipStream_t s, hipEvent_t* ev);
hipError_t launch_route_exact(int fr, int fg, const RouteArgs& a, hipStream_t s, hipEvent_t* ev);
hipError_t launch_exact_experts(int fr, int fs, const DecodeArgs& a, hipStream_t s, hipEvent_t* ev);
hipError_t launch_grouped(int fr, int fs, const GroupedArgs& a, hipStream_t s, hipEvent_t* ev);

}  // namespace moe
