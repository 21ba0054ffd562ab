// Pack loader: validation of layer descriptors, the packed layout, and the
// host repack from the canonical (MLX-style) layout into the kernel layout.
// Pure host code: no HIP call is made here.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <thread>
#include <vector>

#include "moe_host.h"

namespace moe {

static thread_local std::string g_err;

void set_error(const std::string& s) { g_err = s; }
const char* last_error_cstr() { return g_err.c_str(); }

uint64_t align256(uint64_t x) { return (x + 255u) & ~uint64_t(255u); }

std::string fmt_name(const moe_qformat& f) {
  const char* m = f.mode == MOE_AFFINE ? "affine" : f.mode == MOE_SYMMETRIC ? "symmetric"
                : f.mode == MOE_DENSE ? "dense" : f.mode == MOE_MXFP4 ? "mxfp4" : "unknown-mode";
  const char* s = f.scale_dtype == MOE_BF16 ? "bf16" : f.scale_dtype == MOE_FP16 ? "fp16"
                : f.scale_dtype == MOE_E8M0 ? "e8m0" : "unknown-dtype";
  char buf[128];
  snprintf(buf, sizeof buf, "{bits=%d, group=%d, %s, %s}", f.bits, f.group, m, s);
  return buf;
}

static const char* class_name(TensorClass tc) {
  switch (tc) {
    case TC_ROUTER: return "router";
    case TC_GATE_ROW: return "shared-expert gate row";
    case TC_ROUTED: return "routed experts";
    default: return "shared expert";
  }
}

bool format_info(const moe_qformat& f, TensorClass tc, FmtInfo* o) {
  const bool q4 = f.bits == 4 && f.group == 64 && f.mode == MOE_AFFINE && f.scale_dtype == MOE_BF16;
  const bool q3 = f.bits == 3 && f.group == 64 && f.mode == MOE_AFFINE && f.scale_dtype == MOE_BF16;
  const bool q8 = f.bits == 8 && f.group == 64 && f.mode == MOE_AFFINE && f.scale_dtype == MOE_BF16;
  const bool q2 = f.bits == 2 && f.group == 64 && f.mode == MOE_AFFINE && f.scale_dtype == MOE_BF16;
  const bool q5 = f.bits == 5 && f.group == 64 && f.mode == MOE_AFFINE && f.scale_dtype == MOE_BF16;
  const bool q6 = f.bits == 6 && f.group == 64 && f.mode == MOE_AFFINE && f.scale_dtype == MOE_BF16;
  const bool s4 = f.bits == 4 && f.group == 128 && f.mode == MOE_SYMMETRIC && f.scale_dtype == MOE_FP16;
  const bool dn = f.bits == 16 && f.mode == MOE_DENSE && f.scale_dtype == MOE_BF16;
  const bool mx = f.bits == 4 && f.group == 32 && f.mode == MOE_MXFP4 && f.scale_dtype == MOE_E8M0;
  const bool expert = tc == TC_ROUTED || tc == TC_SHARED;
  bool ok = false;
  if (q4) { *o = {KF_Q4, 4, 64, 16, 4, true}; ok = true; }
  else if (q3 && expert) { *o = {KF_Q3, 3, 64, 12, 4, true}; ok = true; }
  else if (q8) { *o = {KF_Q8, 8, 64, 32, 4, true}; ok = true; }
  else if (q2 && expert) { *o = {KF_Q2, 2, 64, 8, 4, true}; ok = true; }
  else if (q5 && expert) { *o = {KF_Q5, 5, 64, 20, 4, true}; ok = true; }
  else if (q6 && expert) { *o = {KF_Q6, 6, 64, 24, 4, true}; ok = true; }
  else if (s4) { *o = {KF_S4, 4, 128, 16, 2, false}; ok = true; }
  else if (dn && tc == TC_GATE_ROW) { *o = {KF_DENSE, 16, 0, 0, 0, false}; ok = true; }
  else if (mx && expert) { *o = {KF_MX4, 4, 32, 16, 1, false}; ok = true; }
  if (!ok) {
    std::string acc = expert ? "{4,64,affine,bf16}, {3,64,affine,bf16}, {8,64,affine,bf16}, {2,64,affine,bf16}, "
                               "{5,64,affine,bf16}, {6,64,affine,bf16}, {4,128,symmetric,fp16}, {4,32,mxfp4,e8m0}"
                     : tc == TC_ROUTER ? "{4,64,affine,bf16}, {8,64,affine,bf16}, {4,128,symmetric,fp16}"
                     : "{4,64,affine,bf16}, {8,64,affine,bf16}, {4,128,symmetric,fp16}, {16,0,dense,bf16}";
    set_error(std::string(class_name(tc)) + " format " + fmt_name(f) +
              " is not read by the kernels; accepted: " + acc);
  }
  return ok;
}

bool grouped_pair_supported(int fr, int fs) {
  const auto low = [](int f) { return f == KF_Q4 || f == KF_Q3 || f == KF_S4; };
  if (low(fr)) return low(fs);
  return (fr == KF_Q2 || fr == KF_Q5 || fr == KF_Q6 || fr == KF_Q8 || fr == KF_MX4) &&
         (fs == fr || fs == KF_Q4);
}

int validate_desc(const moe_layer_desc* d) {
  if (!d) { set_error("layer descriptor is NULL"); return MOE_EINVAL; }
  char buf[256];
  if (d->hidden <= 0 || d->hidden % 256 || d->hidden > 4096) {
    snprintf(buf, sizeof buf, "hidden=%d unsupported: needs a multiple of 256, <= 4096", d->hidden);
    set_error(buf); return MOE_EUNSUPPORTED;
  }
  if (d->n_experts <= 0 || d->n_experts % 64 || d->n_experts > 256) {
    snprintf(buf, sizeof buf, "n_experts=%d unsupported: needs a multiple of 64, <= 256", d->n_experts);
    set_error(buf); return MOE_EUNSUPPORTED;
  }
  if (d->top_k < 1 || d->top_k > 8 || d->top_k > d->n_experts) {
    snprintf(buf, sizeof buf, "top_k=%d unsupported: needs 1..8", d->top_k);
    set_error(buf); return MOE_EUNSUPPORTED;
  }
  if (d->inter <= 0 || d->inter % 256 || d->inter > 2048 ||
      d->shared_inter <= 0 || d->shared_inter % 256 || d->shared_inter > 2048) {
    snprintf(buf, sizeof buf, "inter=%d / shared_inter=%d unsupported: need multiples of 256, <= 2048",
             d->inter, d->shared_inter);
    set_error(buf); return MOE_EUNSUPPORTED;
  }
  if (d->act_dtype != MOE_BF16 && d->act_dtype != MOE_FP16) {
    snprintf(buf, sizeof buf, "act_dtype=%d unsupported: bf16 or fp16", d->act_dtype);
    set_error(buf); return MOE_EUNSUPPORTED;
  }
  FmtInfo fi;
  if (!format_info(d->router, TC_ROUTER, &fi)) return MOE_EUNSUPPORTED;
  if (!format_info(d->gate_row, TC_GATE_ROW, &fi)) return MOE_EUNSUPPORTED;
  if (!format_info(d->routed, TC_ROUTED, &fi)) return MOE_EUNSUPPORTED;
  if (!format_info(d->shared, TC_SHARED, &fi)) return MOE_EUNSUPPORTED;
  // 5- and 6-bit experts: routed and shared of the same width, or routed at
  // 5/6 bits beside a 4-bit affine shared expert (the kernels built for them)
  const int rb = d->routed.bits, sb = d->shared.bits;
  const bool wide_r = rb == 5 || rb == 6, wide_s = sb == 5 || sb == 6;
  const bool q4_s = sb == 4 && d->shared.mode == MOE_AFFINE;
  if ((wide_r || wide_s) && !(rb == sb || (wide_r && q4_s))) {
    snprintf(buf, sizeof buf, "routed %d-bit with shared %d-bit experts unsupported: 5- and 6-bit experts pair "
             "with a shared expert of the same width or 4-bit affine", rb, sb);
    set_error(buf); return MOE_EUNSUPPORTED;
  }
  // MXFP4 experts: routed MXFP4 with an MXFP4 or 4-bit affine shared expert
  const bool mx_r = d->routed.mode == MOE_MXFP4, mx_s = d->shared.mode == MOE_MXFP4;
  if ((mx_r || mx_s) && !(mx_r && (mx_s || q4_s))) {
    set_error("routed " + fmt_name(d->routed) + " with shared " + fmt_name(d->shared) +
              " experts unsupported: MXFP4 routed experts pair with an MXFP4 or 4-bit affine "
              "shared expert");
    return MOE_EUNSUPPORTED;
  }
  return MOE_OK;
}

static uint64_t mat_code_bytes(const FmtInfo& f, uint64_t rows, uint64_t cols) {
  return rows * cols * (uint64_t)f.bits / 8;
}
static uint64_t mat_scale_bytes(const FmtInfo& f, uint64_t rows, uint64_t cols) {
  return rows * (cols / (uint64_t)f.group) * (uint64_t)f.scb;
}

int compute_layout(const moe_layer_desc* d, moe_layer* L) {
  int st = validate_desc(d);
  if (st) return st;
  FmtInfo fr, fg, fe, fs;
  format_info(d->router, TC_ROUTER, &fr);
  format_info(d->gate_row, TC_GATE_ROW, &fg);
  format_info(d->routed, TC_ROUTED, &fe);
  format_info(d->shared, TC_SHARED, &fs);
  const uint64_t H = d->hidden, E = d->n_experts, I = d->inter, Is = d->shared_inter;
  L->d = *d;
  uint64_t off = 0;
  L->router_off = off;
  off = align256(off + mat_code_bytes(fr, E, H));
  L->router_scale_off = off;
  off = align256(off + mat_scale_bytes(fr, E, H));
  L->gate_row_off = off;
  if (fg.kid == KF_DENSE) {
    off = align256(off + H * 2);
    L->gate_row_scale_off = off;
  } else {
    off = align256(off + mat_code_bytes(fg, 1, H));
    L->gate_row_scale_off = off;
    off = align256(off + mat_scale_bytes(fg, 1, H));
  }
  // one expert block: gate/up codes, gate/up scales, down codes, down scales
  auto block = [&](const FmtInfo& f, uint64_t inter, moe_mat_off* gu, moe_mat_off* dn) {
    uint64_t o = 0;
    gu->codes = o; o = align256(o + mat_code_bytes(f, 2 * inter, H));
    gu->scales = o; o = align256(o + mat_scale_bytes(f, 2 * inter, H));
    dn->codes = o; o = align256(o + mat_code_bytes(f, H, inter));
    dn->scales = o; o = align256(o + mat_scale_bytes(f, H, inter));
    return o;
  };
  L->expert_stride = block(fe, I, &L->gu, &L->dn);
  L->experts_off = off;
  off += E * L->expert_stride;
  L->shared_off = off;
  off += block(fs, Is, &L->sh_gu, &L->sh_dn);
  L->bytes = off;
  L->dev = nullptr;
  L->flags = 0;
  return MOE_OK;
}

// True when every E8M0 byte of an MXFP4 tensor's scales (n entries) lies in
// 104..140 or is 255: e2m1 * 2^(e - 127) is then a multiple of 2^(e - 128)
// >= 2^-24 and at most 6 * 2^13 < 65504, exact in fp16 (NaN for 255).
static bool mx_fp16_exact(const moe_qtensor& t, uint64_t n) {
  const uint8_t* e = static_cast<const uint8_t*>(t.scales);
  for (uint64_t i = 0; i < n; ++i)
    if (e[i] != 255 && (e[i] < 104 || e[i] > 140)) return false;
  return true;
}

// ------------------------------------------------------------------ repack
// canonical words covering 32 codes -> kernel words of one lane's chunk
static inline uint32_t q4_word(uint32_t v) {
  uint32_t even = 0, odd = 0;
  for (int j = 0; j < 4; ++j) {
    even |= ((v >> (8 * j)) & 0xFu) << (4 * j);
    odd |= ((v >> (8 * j + 4)) & 0xFu) << (4 * j);
  }
  return even | (odd << 16);
}
static inline uint32_t q8_word(uint32_t v) {
  const uint32_t b0 = v & 0xFF, b1 = (v >> 8) & 0xFF, b2 = (v >> 16) & 0xFF, b3 = v >> 24;
  return b0 | (b2 << 8) | (b1 << 16) | (b3 << 24);
}
// 2-bit: the 16 codes of a canonical word (k = 16w + i), even k in the low
// half and odd k in the high half, pair j at bits 2j and 16 + 2j
static inline uint32_t q2_word(uint32_t v) {
  uint32_t even = 0, odd = 0;
  for (int j = 0; j < 8; ++j) {
    even |= ((v >> (4 * j)) & 3u) << (2 * j);
    odd |= ((v >> (4 * j + 2)) & 3u) << (2 * j);
  }
  return even | (odd << 16);
}
// n bits of a chunk's canonical stream from bit pos (words: the chunk's)
static inline uint32_t stream_bits(const uint32_t* c, int nwords, int pos, int n) {
  const int w = pos / 32, b = pos % 32;
  uint64_t v = c[w];
  if (w + 1 < nwords) v |= (uint64_t)c[w + 1] << 32;
  return (uint32_t)(v >> b) & ((1u << n) - 1u);
}
// 5-bit: pair p < 15 in word p/3 at bits 5 (p mod 3) (and 16 + that); pair 15
// keeps bit b of its codes in bit 15 / bit 31 of word b
static inline void q5_chunk(const uint32_t* c, uint32_t* o) {
  for (int w = 0; w < 5; ++w) o[w] = 0;
  for (int i = 0; i < 32; ++i) {
    const uint32_t q = stream_bits(c, 5, 5 * i, 5);
    const int p = i >> 1, hi = i & 1;
    if (p < 15) {
      o[p / 3] |= q << ((hi ? 16 : 0) + 5 * (p % 3));
    } else {
      for (int b = 0; b < 5; ++b) o[b] |= ((q >> b) & 1u) << (hi ? 31 : 15);
    }
  }
}
// 6-bit: pair p < 12 in word p/2 at bits 6 (p mod 2) (and 16 + that); pair
// 12 + m keeps its low 4 bits in bits 12..15 of word m and its high 2 bits in
// bits 12 + 2 (m mod 2) of word 4 + m/2 (each also at 16 + that for the odd code)
static inline void q6_chunk(const uint32_t* c, uint32_t* o) {
  for (int w = 0; w < 6; ++w) o[w] = 0;
  for (int i = 0; i < 32; ++i) {
    const uint32_t q = stream_bits(c, 6, 6 * i, 6);
    const int p = i >> 1, h = (i & 1) ? 16 : 0;
    if (p < 12) {
      o[p / 2] |= q << (h + 6 * (p % 2));
    } else {
      const int m = p - 12;
      o[m] |= (q & 15u) << (h + 12);
      o[4 + m / 2] |= (q >> 4) << (h + 12 + 2 * (m % 2));
    }
  }
}
static inline void q3_chunk(const uint32_t* c, uint32_t* o) {
  const unsigned __int128 s = (unsigned __int128)c[0] | ((unsigned __int128)c[1] << 32) |
                              ((unsigned __int128)c[2] << 64);
  o[0] = o[1] = o[2] = 0;
  for (int i = 0; i < 32; ++i) {
    const uint32_t q = (uint32_t)(s >> (3 * i)) & 7u;
    const int p = i >> 1, hi = i & 1;
    if (p < 15) {
      o[p / 5] |= q << ((hi ? 16 : 0) + 3 * (p % 5));
    } else {
      for (int b = 0; b < 3; ++b) o[b] |= ((q >> b) & 1u) << (hi ? 31 : 15);
    }
  }
}
static inline void pack_chunk(int kid, const uint32_t* canon, uint32_t* o) {
  switch (kid) {
    case KF_Q4: case KF_S4:
      for (int w = 0; w < 4; ++w) o[w] = q4_word(canon[w]);
      break;
    case KF_Q8:
      for (int w = 0; w < 8; ++w) o[w] = q8_word(canon[w]);
      break;
    case KF_Q3:
      q3_chunk(canon, o);
      break;
    case KF_Q2:
      for (int w = 0; w < 2; ++w) o[w] = q2_word(canon[w]);
      break;
    case KF_Q5:
      q5_chunk(canon, o);
      break;
    case KF_Q6:
      q6_chunk(canon, o);
      break;
    case KF_MX4:
      // byte b of the chunk holds elements 2b (low nibble) and 2b + 1: the
      // canonical words are the kernel's pair order as they stand
      for (int w = 0; w < 4; ++w) o[w] = canon[w];
      break;
  }
}

struct SrcMat {
  const uint32_t* codes;   // [rows, wpr]
  const uint8_t* scales;   // [rows, ng] entries of src_scale_bytes(f) bytes
  const uint16_t* biases;  // [rows, ng] or null
};

// Bytes per source scale entry: bf16 / fp16 2, E8M0 1.
static int src_scale_bytes(const FmtInfo& f) { return f.kid == KF_MX4 ? 1 : 2; }

// Kernel-layout scale entry of group g: affine s | b << 16, else the source
// entry's bytes as they stand.
static void put_scale(const FmtInfo& f, const uint8_t* sr, const uint16_t* br, int g, uint8_t* dst) {
  const int sb = src_scale_bytes(f);
  if (f.affine) {
    uint16_t sv;
    memcpy(&sv, sr + (size_t)g * 2, 2);
    const uint32_t v = (uint32_t)sv | ((uint32_t)br[g] << 16);
    memcpy(dst, &v, 4);
  } else {
    memcpy(dst, sr + (size_t)g * sb, (size_t)sb);
  }
}

// Writes one matrix [O, K] in the tile layout. rowmap(t, lane) -> (which
// source matrix 0/1, source row).
template <class RowMap>
static void pack_matrix(const FmtInfo& f, int O, int K, const SrcMat* srcs, RowMap rowmap,
                        uint8_t* dst_codes, uint8_t* dst_scales) {
  const int ntiles = O / 64, nch = K / 32, nkb = K / 256, gpb = 256 / f.group;
  const int wpr = K * f.bits / 32, ng = K / f.group;
  const int cw = f.bits;  // canonical words per 32-code chunk
  for (int t = 0; t < ntiles; ++t) {
    for (int lane = 0; lane < 64; ++lane) {
      int which, row;
      rowmap(t, lane, &which, &row);
      const SrcMat& s = srcs[which];
      const uint32_t* rw = s.codes + (uint64_t)row * wpr;
      for (int c = 0; c < nch; ++c) {
        uint32_t o[8];
        pack_chunk(f.kid, rw + (uint64_t)c * cw, o);
        uint8_t* blk = dst_codes + ((uint64_t)t * nch + c) * (uint64_t)(64 * f.cb);
        if (f.kid == KF_Q8) {
          memcpy(blk + lane * 16, o, 16);
          memcpy(blk + 64 * 16 + lane * 16, o + 4, 16);
        } else {
          memcpy(blk + lane * f.cb, o, f.cb);
        }
      }
      const uint8_t* sr = s.scales + (uint64_t)row * ng * src_scale_bytes(f);
      const uint16_t* br = s.biases ? s.biases + (uint64_t)row * ng : nullptr;
      for (int kb = 0; kb < nkb; ++kb) {
        uint8_t* sb = dst_scales + (((uint64_t)t * nkb + kb) * 64 + lane) * (uint64_t)(gpb * f.scb);
        for (int gi = 0; gi < gpb; ++gi) put_scale(f, sr, br, kb * gpb + gi, sb + gi * f.scb);
      }
    }
  }
}

static void pack_row(const FmtInfo& f, int K, const moe_qtensor& t, uint8_t* dst_codes,
                     uint8_t* dst_scales) {
  if (f.kid == KF_DENSE) {
    memcpy(dst_codes, t.codes, (size_t)K * 2);
    return;
  }
  const uint32_t* rw = static_cast<const uint32_t*>(t.codes);
  const int nch = K / 32, ng = K / f.group;
  for (int c = 0; c < nch; ++c) {
    uint32_t o[8];
    pack_chunk(f.kid, rw + (uint64_t)c * f.bits, o);
    memcpy(dst_codes + (uint64_t)c * f.cb, o, f.cb);
  }
  for (int g = 0; g < ng; ++g)
    put_scale(f, static_cast<const uint8_t*>(t.scales), t.biases, g, dst_scales + g * f.scb);
}

static bool check_src(const moe_qtensor& t, const FmtInfo& f, const char* name) {
  if (!t.codes || (f.kid != KF_DENSE && !t.scales) || (f.affine && !t.biases)) {
    set_error(std::string("source tensor ") + name + " has a NULL codes/scales/biases pointer");
    return false;
  }
  return true;
}

// Packs gate/up (interleaved per tile) and down of one expert.
static void pack_expert(const FmtInfo& f, int H, int I, const moe_qtensor& g, const moe_qtensor& u,
                        const moe_qtensor& dn, uint64_t e, uint8_t* blk, const moe_mat_off& gu,
                        const moe_mat_off& dno) {
  const uint64_t wg = (uint64_t)I * H * f.bits / 32, sg = (uint64_t)I * (H / f.group);
  const uint64_t wd = (uint64_t)H * I * f.bits / 32, sd = (uint64_t)H * (I / f.group);
  const uint64_t sb = (uint64_t)src_scale_bytes(f);
  const auto sp = [](const moe_qtensor& t) { return static_cast<const uint8_t*>(t.scales); };
  SrcMat gu_src[2] = {
      {static_cast<const uint32_t*>(g.codes) + e * wg, sp(g) + e * sg * sb, g.biases ? g.biases + e * sg : nullptr},
      {static_cast<const uint32_t*>(u.codes) + e * wg, sp(u) + e * sg * sb, u.biases ? u.biases + e * sg : nullptr}};
  pack_matrix(f, 2 * I, H, gu_src,
              [](int t, int lane, int* which, int* row) {
                *which = lane >= 32;
                *row = 32 * t + (lane & 31);
              },
              blk + gu.codes, blk + gu.scales);
  SrcMat d_src[1] = {{static_cast<const uint32_t*>(dn.codes) + e * wd, sp(dn) + e * sd * sb,
                      dn.biases ? dn.biases + e * sd : nullptr}};
  pack_matrix(f, H, I, d_src,
              [](int t, int lane, int* which, int* row) {
                *which = 0;
                *row = 64 * t + lane;
              },
              blk + dno.codes, blk + dno.scales);
}

int pack_layer_host(const moe_layer_desc* d, const moe_layer_src* src, void* host_dst,
                    uint64_t dst_bytes, moe_layer* out) {
  if (!src || !host_dst || !out) { set_error("moe_pack_layer_host: NULL argument"); return MOE_EINVAL; }
  moe_layer L;
  int st = compute_layout(d, &L);
  if (st) return st;
  if (dst_bytes < L.bytes) {
    char buf[160];
    snprintf(buf, sizeof buf, "destination holds %llu bytes, the packed layer needs %llu",
             (unsigned long long)dst_bytes, (unsigned long long)L.bytes);
    set_error(buf);
    return MOE_ENOSPACE;
  }
  FmtInfo fr, fg, fe, fs;
  format_info(d->router, TC_ROUTER, &fr);
  format_info(d->gate_row, TC_GATE_ROW, &fg);
  format_info(d->routed, TC_ROUTED, &fe);
  format_info(d->shared, TC_SHARED, &fs);
  if (!check_src(src->router, fr, "router") || !check_src(src->gate_row, fg, "gate_row") ||
      !check_src(src->gate, fe, "gate") || !check_src(src->up, fe, "up") ||
      !check_src(src->down, fe, "down") || !check_src(src->sh_gate, fs, "sh_gate") ||
      !check_src(src->sh_up, fs, "sh_up") || !check_src(src->sh_down, fs, "sh_down"))
    return MOE_EINVAL;
  uint8_t* base = static_cast<uint8_t*>(host_dst);
  memset(base, 0, L.bytes);
  const int H = d->hidden, E = d->n_experts, I = d->inter, Is = d->shared_inter;
  SrcMat rsrc[1] = {{static_cast<const uint32_t*>(src->router.codes), static_cast<const uint8_t*>(src->router.scales),
                     src->router.biases}};
  pack_matrix(fr, E, H, rsrc,
              [](int t, int lane, int* which, int* row) { *which = 0; *row = 64 * t + lane; },
              base + L.router_off, base + L.router_scale_off);
  pack_row(fg, H, src->gate_row, base + L.gate_row_off, base + L.gate_row_scale_off);
  // routed experts in parallel (independent blocks)
  unsigned nt = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  std::vector<std::thread> th;
  for (unsigned w = 0; w < nt; ++w) {
    th.emplace_back([&, w]() {
      for (int e = (int)w; e < E; e += (int)nt)
        pack_expert(fe, H, I, src->gate, src->up, src->down, (uint64_t)e,
                    base + L.experts_off + (uint64_t)e * L.expert_stride, L.gu, L.dn);
    });
  }
  for (auto& t : th) t.join();
  pack_expert(fs, H, Is, src->sh_gate, src->sh_up, src->sh_down, 0, base + L.shared_off, L.sh_gu,
              L.sh_dn);
  if (fe.kid == KF_MX4 || fs.kid == KF_MX4) {
    bool ok = true;
    if (fe.kid == KF_MX4) {
      const uint64_t n = (uint64_t)E * I * (H / 32);
      ok = mx_fp16_exact(src->gate, n) && mx_fp16_exact(src->up, n) && mx_fp16_exact(src->down, n);
    }
    if (ok && fs.kid == KF_MX4) {
      const uint64_t n = (uint64_t)Is * (H / 32);
      ok = mx_fp16_exact(src->sh_gate, n) && mx_fp16_exact(src->sh_up, n) && mx_fp16_exact(src->sh_down, n);
    }
    if (ok) L.flags |= MOE_LAYER_MX_FP16;
  }
  *out = L;
  return MOE_OK;
}

RouteWs route_ws_layout(const moe_layer_desc* d, int rows) {
  RouteWs w;
  uint64_t o = 0;
  // the decode router's hand-off words (32 rows x 32 entries) and its call
  // counter words: one fixed area at the start whatever the row count of the
  // call, so no other part of any call's workspace overlaps it
  w.cand_off = o; o = align256(o + 32 * 32 * 8);
  w.sync_off = o; o = align256(o + 16);
  w.gl_off = o; o = align256(o + (uint64_t)rows * 4);
  w.lg_off = o; o = align256(o + (uint64_t)rows * d->n_experts * 4);
  w.total = o;
  return w;
}

uint64_t route_ws_bytes(const moe_layer_desc* d, int rows) { return route_ws_layout(d, rows).total; }

DecodeWs decode_ws_layout(const moe_layer_desc* d, int rows) {
  const uint64_t Imax = std::max(d->inter, d->shared_inter);
  const uint64_t slots = (uint64_t)rows * (d->top_k + 1);
  DecodeWs w;
  uint64_t o = route_ws_bytes(d, rows);
  w.hhi_off = o; o = align256(o + slots * Imax * 2);
  w.hlo_off = o; o = align256(o + slots * Imax * 2);
  w.hc_off = o; o = align256(o + slots * (Imax / 32) * 4);
  w.total = o;
  return w;
}

ExactWs exact_ws_layout(const moe_layer_desc* d, int rows) {
  const uint64_t E = d->n_experts, slots = (uint64_t)rows * (d->top_k + 1);
  ExactWs w;
  w.dec = decode_ws_layout(d, rows);
  uint64_t o = w.dec.total;
  w.meta_off = o; o = align256(o + (E + 16) * 4);
  w.perm_off = o; o = align256(o + slots * 4);
  // an expert's run of c rows is ceil(c / 16) blocks: at most slots/16 + E + 1
  w.max_blocks = (int)(slots / 16 + E + 2);
  w.blocks_off = o; o = align256(o + (uint64_t)w.max_blocks * 3 * 4);
  w.e_off = o; o = align256(o + slots * d->hidden * 4);
  w.total = o;
  return w;
}

GroupedWs grouped_ws_layout(const moe_layer_desc* d, int rows) {
  const uint64_t E = d->n_experts, k = d->top_k, H = d->hidden;
  const uint64_t Imax = std::max(d->inter, d->shared_inter);
  const uint64_t slots = (uint64_t)rows * (k + 1);
  GroupedWs w;
  uint64_t o = route_ws_bytes(d, rows);
  w.meta_off = o; o = align256(o + (8 + E + 2) * 4);
  w.perm_off = o; o = align256(o + slots * 4);
  w.h_off = o; o = align256(o + slots * Imax * 2);
  w.e_off = o; o = align256(o + slots * H * 4);
  w.x16_off = o; o = align256(o + (uint64_t)rows * H * 2);
  // work list: an expert's rows split into M-tiles of 128 rows and one
  // shorter last tile: at most slots/128 + E + 1 tiles
  w.max_tiles = (int)(slots / 128 + E + 2);
  w.tiles_off = o; o = align256(o + (uint64_t)w.max_tiles * 3 * 4);
  w.total = o;
  return w;
}

}  // namespace moe
