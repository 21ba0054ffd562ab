// Host-side internals shared by the pack loader and the entry points.
#pragma once
#include <stdint.h>

#include <string>

#include "../../include/moe.h"

namespace moe {

// kernel-side format ids (match moe_kernels.h)
enum { KF_Q4 = 0, KF_Q3 = 1, KF_Q8 = 2, KF_S4 = 3, KF_DENSE = 4, KF_Q2 = 5, KF_Q5 = 6, KF_Q6 = 7, KF_MX4 = 8 };

struct FmtInfo {
  int kid;      // kernel format id
  int bits;     // code width (16 for dense)
  int group;    // group size (0 for dense)
  int cb;       // bytes per lane per 32-code chunk
  int scb;      // bytes per group scale entry in the kernel layout
  bool affine;
};

// Tensor classes, for messages and accepted-format tables.
enum TensorClass { TC_ROUTER = 0, TC_GATE_ROW, TC_ROUTED, TC_SHARED };

// Returns false (and sets the thread-local error naming the class) when the
// format is not read by the kernels for that tensor class.
bool format_info(const moe_qformat& f, TensorClass tc, FmtInfo* out);
// The routed / shared format pair (KF_ ids) the grouped GEMMs read: the 3-
// and 4-bit formats in any pairing, the 2-, 5-, 6-, 8-bit and MXFP4 ones with
// a shared expert of the same format or 4-bit affine.
bool grouped_pair_supported(int fr, int fs);

// Validates a descriptor (shapes + formats). Sets the error on failure.
int validate_desc(const moe_layer_desc* d);

// Computes every offset of the packed layout into *out (out->dev untouched).
int compute_layout(const moe_layer_desc* d, moe_layer* out);

void set_error(const std::string& s);
std::string fmt_name(const moe_qformat& f);

uint64_t align256(uint64_t x);

// Route scratch at the start of every workspace: the decode router's
// hand-off words and their call-counter words (a fixed area, kept consistent
// by every call), gate-row logits, then [rows, E] fp32 logits.
struct RouteWs {
  uint64_t cand_off, sync_off, gl_off, lg_off, total;
};
RouteWs route_ws_layout(const moe_layer_desc* d, int rows);
uint64_t route_ws_bytes(const moe_layer_desc* d, int rows);

// Workspace layout of the decode path (after the route scratch).
struct DecodeWs {
  uint64_t hhi_off, hlo_off, hc_off, total;
};
DecodeWs decode_ws_layout(const moe_layer_desc* d, int rows);

// Per-kind workspace layout of the grouped path.
struct GroupedWs {
  uint64_t meta_off;   // after the route scratch: int32 tile counts, offsets[E+2]
  uint64_t perm_off;   // int32 [R*k + R]: expert-major position -> slot index (r*(k+1)+j)
  uint64_t h_off;      // f16 [R*(k+1), Imax] in expert-major order
  uint64_t e_off;      // f32 [R*(k+1), H] in slot order (r*(k+1)+j)
  uint64_t x16_off;    // f16 [R, H] activations for the GEMMs (bf16 layers)
  uint64_t tiles_off;  // int32 [max_tiles][3] work list of M-tiles
  uint64_t total;
  int max_tiles;
};
GroupedWs grouped_ws_layout(const moe_layer_desc* d, int rows);

// Workspace layout of the exact chunk form (moe_forward_exact): the decode
// layout for all rows (route scratch with [rows, E] logits, then the h
// parts of every slot), then the sort's arrays and its list of expert blocks.
struct ExactWs {
  DecodeWs dec;
  uint64_t meta_off;     // int32: block count, queue words, expert offsets [E+2]
  uint64_t perm_off;     // int32 [R*(k+1)]: expert-major position -> slot index r*(k+1)+j
  uint64_t blocks_off;   // int32 [max_blocks][3]: (expert, first position, rows <= 16)
  uint64_t e_off;        // f32 [R*(k+1), H]: slot outputs of down, in slot order
  uint64_t total;
  int max_blocks;
};
ExactWs exact_ws_layout(const moe_layer_desc* d, int rows);

// moe_forward_windows with the router's sticky-failure rule switchable
// (sticky = 0: a failure recorded in the workspace by an earlier call does
// not mark this call's rows).
int forward_windows_impl(const moe_layer* layer, const void* x, int rows, const float* logit_bias,
                         int32_t* ids, float* p, float* shared_gate, float* y, void* ws,
                         uint64_t ws_bytes, void* stream, int sticky);

}  // namespace moe
