// C entry points: argument validation, then the kernel launches.
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "moe_host.h"
#include "moe_launch.h"

namespace moe {
const char* last_error_cstr();
int pack_layer_host(const moe_layer_desc* d, const moe_layer_src* src, void* host_dst,
                    uint64_t dst_bytes, moe_layer* out);
}  // namespace moe

using namespace moe;

static int hip_fail(const char* what, hipError_t e) {
  set_error(std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")");
  return MOE_EHIP;
}

static int check_layer(const moe_layer* L) {
  if (!L) { set_error("layer is NULL"); return MOE_EINVAL; }
  if (!L->dev) { set_error("layer has no device buffer (moe_layer_bind was not called)"); return MOE_EINVAL; }
  int st = validate_desc(&L->d);
  if (st) return st;
  moe_layer ref;
  compute_layout(&L->d, &ref);
  if (ref.bytes != L->bytes || ref.experts_off != L->experts_off || ref.shared_off != L->shared_off) {
    set_error("layer offsets do not match its descriptor (not produced by this library version)");
    return MOE_ESHAPE;
  }
  return MOE_OK;
}

static hipEvent_t* taps_events(const moe_taps* taps) {
  return taps ? reinterpret_cast<hipEvent_t*>(const_cast<void**>(taps->kernel_events)) : nullptr;
}

static ExpertClass expert_class(const moe_layer* L, bool shared) {
  ExpertClass c;
  if (shared) {
    c.base_off = L->shared_off;
    c.stride = 0;
    c.gu_codes = L->sh_gu.codes;
    c.gu_scales = L->sh_gu.scales;
    c.dn_codes = L->sh_dn.codes;
    c.dn_scales = L->sh_dn.scales;
    c.blk_bytes = (uint32_t)(L->bytes - L->shared_off);
    c.inter = L->d.shared_inter;
  } else {
    c.base_off = L->experts_off;
    c.stride = L->expert_stride;
    c.gu_codes = L->gu.codes;
    c.gu_scales = L->gu.scales;
    c.dn_codes = L->dn.codes;
    c.dn_scales = L->dn.scales;
    c.blk_bytes = (uint32_t)L->expert_stride;
    c.inter = L->d.inter;
  }
  return c;
}

extern "C" {

int moe_pack_size(const moe_layer_desc* d, uint64_t* bytes) {
  if (!d || !bytes) { set_error("moe_pack_size: NULL argument"); return MOE_EINVAL; }
  moe_layer L;
  int st = compute_layout(d, &L);
  if (st) return st;
  *bytes = L.bytes;
  return MOE_OK;
}

int moe_pack_layer_host(const moe_layer_desc* d, const moe_layer_src* src, void* host_dst,
                        uint64_t dst_bytes, moe_layer* out) {
  return pack_layer_host(d, src, host_dst, dst_bytes, out);
}

int moe_layer_bind(moe_layer* layer, const void* dev_ptr) {
  if (!layer || !dev_ptr) { set_error("moe_layer_bind: NULL argument"); return MOE_EINVAL; }
  if (reinterpret_cast<uintptr_t>(dev_ptr) & 255u) {
    set_error("moe_layer_bind: device pointer is not 256-byte aligned");
    return MOE_EINVAL;
  }
  layer->dev = dev_ptr;
  return MOE_OK;
}

int moe_pack_layer(const moe_layer_desc* d, const moe_layer_src* src, void* dev_dst,
                   uint64_t dst_bytes, void* stream, moe_layer* out) {
  if (!dev_dst || !out) { set_error("moe_pack_layer: NULL argument"); return MOE_EINVAL; }
  uint64_t bytes = 0;
  int st = moe_pack_size(d, &bytes);
  if (st) return st;
  if (dst_bytes < bytes) {
    set_error("moe_pack_layer: device destination smaller than moe_pack_size");
    return MOE_ENOSPACE;
  }
  std::vector<uint8_t> host(bytes);
  moe_layer L;
  st = pack_layer_host(d, src, host.data(), bytes, &L);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(dev_dst, host.data(), bytes, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail("moe_pack_layer: hipMemcpyAsync", e);
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail("moe_pack_layer: hipStreamSynchronize", e);
  st = moe_layer_bind(&L, dev_dst);
  if (st) return st;
  *out = L;
  return MOE_OK;
}

int moe_workspace_size(const moe_layer_desc* d, int rows, int grouped, uint64_t* bytes) {
  if (!d || !bytes) { set_error("moe_workspace_size: NULL argument"); return MOE_EINVAL; }
  int st = validate_desc(d);
  if (st) return st;
  if (grouped < MOE_WS_DECODE || grouped > MOE_WS_EXACT) {
    set_error("moe_workspace_size: kind " + std::to_string(grouped) + " is not MOE_WS_DECODE, MOE_WS_GROUPED "
              "or MOE_WS_EXACT");
    return MOE_EINVAL;
  }
  if (rows < 1 || (grouped == MOE_WS_DECODE && rows > 16) || rows > 65536) {
    set_error(std::string("moe_workspace_size: rows=") + std::to_string(rows) +
              (grouped != MOE_WS_DECODE ? " outside 1..65536" : " outside 1..16 (decode)"));
    return MOE_EINVAL;
  }
  *bytes = grouped == MOE_WS_GROUPED ? grouped_ws_layout(d, rows).total
           : grouped == MOE_WS_EXACT ? exact_ws_layout(d, rows).total
                                     : decode_ws_layout(d, rows).total;
  return MOE_OK;
}

static constexpr int kWindowRows = 16;   // decode rows per window of moe_forward_windows

// moe_route; sticky = 0 keeps an earlier failure recorded in the workspace
// from marking this call's rows (the static-scratch entry point, whose
// callers cannot clear the count).
static int route_impl(const moe_layer* layer, const void* x, int rows, const float* logit_bias,
                      int32_t* ids, float* p, float* shared_gate, void* ws, uint64_t ws_bytes,
                      const moe_taps* taps, void* stream, int sticky) {
  int st = check_layer(layer);
  if (st) return st;
  if (!x || !ids || !p || !shared_gate || !ws) {
    set_error("moe_route: NULL x/ids/p/shared_gate/ws");
    return MOE_EINVAL;
  }
  if (rows < 1 || rows > 65536) { set_error("moe_route: rows outside 1..65536"); return MOE_EINVAL; }
  if (ws_bytes < route_ws_bytes(&layer->d, rows)) {
    set_error("moe_route: workspace of " + std::to_string(ws_bytes) + " bytes, needs " +
              std::to_string(route_ws_bytes(&layer->d, rows)));
    return MOE_ENOSPACE;
  }
  FmtInfo fr, fg;
  format_info(layer->d.router, TC_ROUTER, &fr);
  format_info(layer->d.gate_row, TC_GATE_ROW, &fg);
  RouteArgs a{};
  a.base = static_cast<const uint8_t*>(layer->dev);
  a.r_off = layer->router_off;
  a.r_soff = layer->router_scale_off;
  a.g_off = layer->gate_row_off;
  a.g_soff = layer->gate_row_scale_off;
  a.x = static_cast<const uint16_t*>(x);
  a.act_fp16 = layer->d.act_dtype == MOE_FP16;
  a.H = layer->d.hidden;
  a.E = layer->d.n_experts;
  a.k = layer->d.top_k;
  a.bias = logit_bias;
  a.ids = ids;
  a.p = p;
  a.sg = shared_gate;
  a.R = rows;
  a.logits = taps ? taps->logits : nullptr;
  a.wait_limit = (taps && taps->route_wait_limit < 0) ? 0 : (1 << 22);
  a.sticky = sticky;
  const RouteWs rw = route_ws_layout(&layer->d, rows);
  uint8_t* wb = static_cast<uint8_t*>(ws);
  a.lg_ws = reinterpret_cast<float*>(wb + rw.lg_off);
  a.gl_ws = reinterpret_cast<float*>(wb + rw.gl_off);
  a.cand = reinterpret_cast<uint64_t*>(wb + rw.cand_off);
  a.sync = reinterpret_cast<uint32_t*>(wb + rw.sync_off);
  hipError_t e = launch_route(fr.kid, fg.kid, a, static_cast<hipStream_t>(stream), taps_events(taps));
  if (e != hipSuccess) return hip_fail("moe_route: launch", e);
  return MOE_OK;
}

int moe_route(const moe_layer* layer, const void* x, int rows, const float* logit_bias,
              int32_t* ids, float* p, float* shared_gate, void* ws, uint64_t ws_bytes,
              const moe_taps* taps, void* stream) {
  return route_impl(layer, x, rows, logit_bias, ids, p, shared_gate, ws, ws_bytes, taps, stream, 1);
}

static int experts_common(const char* name, const moe_layer* layer, const void* x, int rows,
                          const int32_t* ids, const float* p, const float* sg, float* y,
                          void* ws, int max_rows) {
  int st = check_layer(layer);
  if (st) return st;
  if (!x || !ids || !p || !sg || !y || !ws) {
    set_error(std::string(name) + ": NULL x/ids/p/shared_gate/y/ws");
    return MOE_EINVAL;
  }
  if (rows < 1 || rows > max_rows) {
    set_error(std::string(name) + ": rows=" + std::to_string(rows) + " outside 1.." +
              std::to_string(max_rows));
    return MOE_EINVAL;
  }
  return MOE_OK;
}

int moe_experts_decode(const moe_layer* layer, const void* x, int rows, const int32_t* ids,
                       const float* p, const float* shared_gate, float* y, void* ws,
                       uint64_t ws_bytes, const moe_taps* taps, void* stream) {
  int st = experts_common("moe_experts_decode", layer, x, rows, ids, p, shared_gate, y, ws, 16);
  if (st) return st;
  const DecodeWs wl = decode_ws_layout(&layer->d, rows);
  if (ws_bytes < wl.total) {
    set_error("moe_experts_decode: workspace of " + std::to_string(ws_bytes) + " bytes, needs " +
              std::to_string(wl.total));
    return MOE_ENOSPACE;
  }
  FmtInfo fe, fs;
  format_info(layer->d.routed, TC_ROUTED, &fe);
  format_info(layer->d.shared, TC_SHARED, &fs);
  DecodeArgs a{};
  a.base = static_cast<const uint8_t*>(layer->dev);
  a.rt = expert_class(layer, false);
  a.sh = expert_class(layer, true);
  a.x = static_cast<const uint16_t*>(x);
  a.act_fp16 = layer->d.act_dtype == MOE_FP16;
  a.H = layer->d.hidden;
  a.E = layer->d.n_experts;
  a.k = layer->d.top_k;
  a.R = rows;
  a.Imax = std::max(layer->d.inter, layer->d.shared_inter);
  a.ids = ids;
  a.p = p;
  a.sg = shared_gate;
  uint8_t* w = static_cast<uint8_t*>(ws);
  a.hhi = reinterpret_cast<uint16_t*>(w + wl.hhi_off);
  a.hlo = reinterpret_cast<uint16_t*>(w + wl.hlo_off);
  a.hc = reinterpret_cast<float*>(w + wl.hc_off);
  a.y = y;
  a.tap_gu = taps ? taps->gu : nullptr;
  a.tap_h = taps ? taps->h : nullptr;
  a.tap_e = taps ? taps->e : nullptr;
  hipError_t e = launch_decode(fe.kid, fs.kid, a, static_cast<hipStream_t>(stream), taps_events(taps));
  if (e != hipSuccess) return hip_fail("moe_experts_decode: launch", e);
  return MOE_OK;
}

}  // extern "C"

int moe::forward_windows_impl(const moe_layer* layer, const void* x, int rows, const float* logit_bias,
                              int32_t* ids, float* p, float* shared_gate, float* y, void* ws,
                              uint64_t ws_bytes, void* stream, int sticky) {
  int st = check_layer(layer);
  if (st) return st;
  if (!x || !ids || !p || !shared_gate || !y || !ws) {
    set_error("moe_forward_windows: NULL x/ids/p/shared_gate/y/ws");
    return MOE_EINVAL;
  }
  if (rows < 1 || rows > 65536) { set_error("moe_forward_windows: rows outside 1..65536"); return MOE_EINVAL; }
  // every window needs at most a 16-row decode workspace; checked before
  // anything is enqueued
  const int wmax = std::min(rows, kWindowRows);
  const uint64_t need = decode_ws_layout(&layer->d, wmax).total;
  if (ws_bytes < need) {
    set_error("moe_forward_windows: workspace of " + std::to_string(ws_bytes) + " bytes, needs " +
              std::to_string(need));
    return MOE_ENOSPACE;
  }
  const int H = layer->d.hidden, k = layer->d.top_k;
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  for (int r0 = 0; r0 < rows; r0 += kWindowRows) {
    const int n = std::min(kWindowRows, rows - r0);
    const void* xw = xb + (uint64_t)r0 * H * 2;
    int32_t* iw = ids + (uint64_t)r0 * k;
    float* pw = p + (uint64_t)r0 * k;
    float* sw = shared_gate + r0;
    st = route_impl(layer, xw, n, logit_bias, iw, pw, sw, ws, ws_bytes, nullptr, stream, sticky);
    if (st) return st;
    st = moe_experts_decode(layer, xw, n, iw, pw, sw, y + (uint64_t)r0 * H, ws, ws_bytes, nullptr, stream);
    if (st) return st;
  }
  return MOE_OK;
}

extern "C" {

int moe_forward_windows(const moe_layer* layer, const void* x, int rows, const float* logit_bias,
                        int32_t* ids, float* p, float* shared_gate, float* y, void* ws, uint64_t ws_bytes,
                        void* stream) {
  return forward_windows_impl(layer, x, rows, logit_bias, ids, p, shared_gate, y, ws, ws_bytes, stream, 1);
}

int moe_forward_exact(const moe_layer* layer, const void* x, int rows, const float* logit_bias, int32_t* ids,
                      float* p, float* shared_gate, float* y, void* ws, uint64_t ws_bytes, const moe_taps* taps,
                      void* stream) {
  int st = check_layer(layer);
  if (st) return st;
  if (!x || !ids || !p || !shared_gate || !y || !ws) {
    set_error("moe_forward_exact: NULL x/ids/p/shared_gate/y/ws");
    return MOE_EINVAL;
  }
  if (rows < 1 || rows > 65536) { set_error("moe_forward_exact: rows outside 1..65536"); return MOE_EINVAL; }
  const moe_layer_desc* d = &layer->d;
  const ExactWs wl = exact_ws_layout(d, rows);
  if (ws_bytes < wl.total) {
    set_error("moe_forward_exact: workspace of " + std::to_string(ws_bytes) + " bytes, needs " +
              std::to_string(wl.total) + " (moe_workspace_size with MOE_WS_EXACT)");
    return MOE_ENOSPACE;
  }
  FmtInfo fr, fg, fe, fs;
  format_info(d->router, TC_ROUTER, &fr);
  format_info(d->gate_row, TC_GATE_ROW, &fg);
  format_info(d->routed, TC_ROUTED, &fe);
  format_info(d->shared, TC_SHARED, &fs);
  if (d->shared_inter / fs.group > 32) {
    // the down kernel keeps at most 32 shared-expert group values per row
    set_error("moe_forward_exact: shared expert " + fmt_name(d->shared) + " with shared_inter=" +
              std::to_string(d->shared_inter) + " has more than 32 groups per row (moe_forward_windows "
              "reads it)");
    return MOE_EUNSUPPORTED;
  }
  uint8_t* w = static_cast<uint8_t*>(ws);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t* ev = taps_events(taps);
  // 1. the router with the decode router's per-row arithmetic
  RouteArgs ra{};
  ra.base = static_cast<const uint8_t*>(layer->dev);
  ra.r_off = layer->router_off;
  ra.r_soff = layer->router_scale_off;
  ra.g_off = layer->gate_row_off;
  ra.g_soff = layer->gate_row_scale_off;
  ra.x = static_cast<const uint16_t*>(x);
  ra.act_fp16 = d->act_dtype == MOE_FP16;
  ra.H = d->hidden;
  ra.E = d->n_experts;
  ra.k = d->top_k;
  ra.bias = logit_bias;
  ra.ids = ids;
  ra.p = p;
  ra.sg = shared_gate;
  ra.R = rows;
  ra.logits = taps ? taps->logits : nullptr;
  const RouteWs rw = route_ws_layout(d, rows);
  ra.lg_ws = reinterpret_cast<float*>(w + rw.lg_off);
  ra.gl_ws = reinterpret_cast<float*>(w + rw.gl_off);
  ra.cand = reinterpret_cast<uint64_t*>(w + rw.cand_off);
  ra.sync = reinterpret_cast<uint32_t*>(w + rw.sync_off);
  hipError_t e = launch_route_exact(fr.kid, fg.kid, ra, s, ev);
  if (e != hipSuccess) return hip_fail("moe_forward_exact: route launch", e);
  // 2. the slots in expert-major order and the expert blocks of 16 rows
  GroupedArgs ga{};
  ga.E = d->n_experts;
  ga.k = d->top_k;
  ga.R = rows;
  ga.H = d->hidden;
  ga.ids = ids;
  ga.meta = reinterpret_cast<int32_t*>(w + wl.meta_off);
  ga.perm = reinterpret_cast<int32_t*>(w + wl.perm_off);
  ga.tiles = reinterpret_cast<int32_t*>(w + wl.blocks_off);
  ga.max_tiles = wl.max_blocks;
  ga.blk16 = 1;
  e = launch_grp_sort(ga, s, ev ? ev + 2 : nullptr);
  if (e != hipSuccess) return hip_fail("moe_forward_exact: sort launch", e);
  // 3. gate/up on the blocks, then the decode down + combine of every row
  DecodeArgs da{};
  da.base = static_cast<const uint8_t*>(layer->dev);
  da.rt = expert_class(layer, false);
  da.sh = expert_class(layer, true);
  da.x = static_cast<const uint16_t*>(x);
  da.act_fp16 = d->act_dtype == MOE_FP16;
  da.H = d->hidden;
  da.E = d->n_experts;
  da.k = d->top_k;
  da.R = rows;
  da.Imax = std::max(d->inter, d->shared_inter);
  da.ids = ids;
  da.p = p;
  da.sg = shared_gate;
  da.hhi = reinterpret_cast<uint16_t*>(w + wl.dec.hhi_off);
  da.hlo = reinterpret_cast<uint16_t*>(w + wl.dec.hlo_off);
  da.hc = reinterpret_cast<float*>(w + wl.dec.hc_off);
  da.y = y;
  da.tap_gu = taps ? taps->gu : nullptr;
  da.tap_h = taps ? taps->h : nullptr;
  da.tap_e = taps ? taps->e : nullptr;
  da.perm = ga.perm;
  da.blocks = ga.tiles;
  da.nblocks = ga.meta;
  da.e_ws = reinterpret_cast<float*>(w + wl.e_off);
  e = launch_exact_experts(fe.kid, fs.kid, da, s, ev ? ev + 4 : nullptr);
  if (e != hipSuccess) return hip_fail("moe_forward_exact: experts launch", e);
  return MOE_OK;
}

int moe_experts_grouped(const moe_layer* layer, const void* x, int rows, const int32_t* ids,
                        const float* p, const float* shared_gate, float* y, void* ws,
                        uint64_t ws_bytes, const moe_taps* taps, void* stream) {
  int st = experts_common("moe_experts_grouped", layer, x, rows, ids, p, shared_gate, y, ws, 65536);
  if (st) return st;
  {
    // the grouped GEMMs read the 3- and 4-bit formats in any pairing and
    // the 2-, 5-, 6- and 8-bit ones with a shared expert of the same width
    // or 4-bit affine
    FmtInfo fr, fs;
    if (!format_info(layer->d.routed, TC_ROUTED, &fr) || !format_info(layer->d.shared, TC_SHARED, &fs))
      return MOE_EUNSUPPORTED;
    if (!grouped_pair_supported(fr.kid, fs.kid)) {
      set_error("moe_experts_grouped: routed " + fmt_name(layer->d.routed) + " with shared " +
                fmt_name(layer->d.shared) + " is not read by the grouped GEMMs (a 2-, 5-, 6-, 8-bit or MXFP4 "
                "routed format needs a shared expert of the same format or 4-bit affine); moe_forward_windows "
                "reads it");
      return MOE_EUNSUPPORTED;
    }
    if ((fr.kid == KF_MX4 || fs.kid == KF_MX4) && !(layer->flags & MOE_LAYER_MX_FP16)) {
      set_error("moe_experts_grouped: MXFP4 experts whose block exponents leave 104..140 (or a layer not "
                "packed by moe_pack_layer_host) are not exact in the grouped GEMMs' fp16 operands; "
                "moe_forward_windows and moe_forward_exact read them");
      return MOE_EUNSUPPORTED;
    }
  }
  const GroupedWs wl = grouped_ws_layout(&layer->d, rows);
  if (ws_bytes < wl.total) {
    set_error("moe_experts_grouped: workspace of " + std::to_string(ws_bytes) + " bytes, needs " +
              std::to_string(wl.total));
    return MOE_ENOSPACE;
  }
  FmtInfo fe, fs;
  format_info(layer->d.routed, TC_ROUTED, &fe);
  format_info(layer->d.shared, TC_SHARED, &fs);
  GroupedArgs a{};
  a.base = static_cast<const uint8_t*>(layer->dev);
  a.rt = expert_class(layer, false);
  a.sh = expert_class(layer, true);
  a.x = static_cast<const uint16_t*>(x);
  a.act_fp16 = layer->d.act_dtype == MOE_FP16;
  a.H = layer->d.hidden;
  a.E = layer->d.n_experts;
  a.k = layer->d.top_k;
  a.R = rows;
  a.Imax = std::max(layer->d.inter, layer->d.shared_inter);
  a.ids = ids;
  a.p = p;
  a.sg = shared_gate;
  uint8_t* w = static_cast<uint8_t*>(ws);
  a.meta = reinterpret_cast<int32_t*>(w + wl.meta_off);
  a.perm = reinterpret_cast<int32_t*>(w + wl.perm_off);
  a.hbuf = reinterpret_cast<uint16_t*>(w + wl.h_off);
  a.e_ws = reinterpret_cast<float*>(w + wl.e_off);
  a.tiles = reinterpret_cast<int32_t*>(w + wl.tiles_off);
  a.max_tiles = wl.max_tiles;
  a.x16 = a.act_fp16 ? a.x : reinterpret_cast<const uint16_t*>(w + wl.x16_off);
  a.y = y;
  a.tap_gu = taps ? taps->gu : nullptr;
  a.tap_h = taps ? taps->h : nullptr;
  a.tap_e = taps ? taps->e : nullptr;
  hipError_t e = launch_grouped(fe.kid, fs.kid, a, static_cast<hipStream_t>(stream), taps_events(taps));
  if (e != hipSuccess) return hip_fail("moe_experts_grouped: launch", e);
  return MOE_OK;
}

int moe_route_failures(void* ws, uint64_t ws_bytes, int clear, uint32_t* count, void* stream) {
  if (!ws || !count) { set_error("moe_route_failures: NULL ws/count"); return MOE_EINVAL; }
  moe_layer_desc d{};
  d.n_experts = 64;
  const RouteWs rw = route_ws_layout(&d, 1);
  if (ws_bytes < rw.sync_off + 16) {
    set_error("moe_route_failures: workspace smaller than its fixed router area");
    return MOE_ENOSPACE;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* word = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + rw.sync_off) + 2;
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, word, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail("moe_route_failures: read", e);
  if (clear && v != 0) {
    e = hipMemsetAsync(word, 0, 4, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail("moe_route_failures: clear", e);
  }
  *count = v;
  return MOE_OK;
}

const char* moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: format or shape not read by the kernels";
    case MOE_ESHAPE: return "MOE_ESHAPE: inconsistent shapes";
    case MOE_ENOSPACE: return "MOE_ENOSPACE: buffer too small";
    case MOE_EHIP: return "MOE_EHIP: HIP runtime error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return last_error_cstr(); }

const char* moe_version(void) { return "moe-mi355x 0.1 (gfx950)"; }

}  // extern "C"
