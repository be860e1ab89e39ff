// C-ABI entry points of libtwell: argument checks on the host, then kernel
// launches on the caller's stream.  No allocation, no synchronisation.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>
#include <mutex>

#include "../../include/twell.h"
#include "internal.hpp"

using namespace twell;

namespace {

thread_local char g_err[512] = "";

twell_status fail(twell_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

twell_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return TWELL_OK;
  return fail(TWELL_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr int GPU_R = 16, GPU_C = 64;

// Carves consecutive 256-byte aligned regions out of a workspace.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off = round_up(off + bytes, 256);
    return p;
  }
};

void mat_parts(int64_t T, int64_t F, int64_t R, int64_t C, twell_dtype v, size_t parts[5]) {
  const int64_t NR = (T + R - 1) / R, NT = (F + C - 1) / C;
  parts[0] = (size_t)(T * NT);
  parts[1] = (size_t)(NR * NT);
  parts[2] = (size_t)(NR * NT * C * R) * (v == TWELL_F32 ? 4 : 2);
  parts[3] = (size_t)(NR * NT * C * R);
  parts[4] = (size_t)(T * NT) * 8;
}

twell_status check_shape(const twell_ffn_shape* sh) {
  if (!sh) return fail(TWELL_EINVAL, "shape is NULL");
  if (sh->T < 0 || sh->d <= 0 || sh->F <= 0) return fail(TWELL_EINVAL, "bad shape T=%d d=%d F=%d", sh->T, sh->d, sh->F);
  if ((sh->in_dt != TWELL_F32 && sh->in_dt != TWELL_BF16) || (sh->out_dt != TWELL_F32 && sh->out_dt != TWELL_BF16))
    return fail(TWELL_EINVAL, "bad dtype");
  if (sh->d % 64 != 0 || sh->F % 64 != 0)
    return fail(TWELL_EUNSUPPORTED, "GPU path needs d %% 64 == 0 and F %% 64 == 0 (d=%d F=%d)", sh->d, sh->F);
  if (sh->F > 65472) return fail(TWELL_EUNSUPPORTED, "F=%d too large (max 65472)", sh->F);
  // The GEMM mainloops address a 16-bit operand ([T][d] activations, [F][d]
  // weights, the [T][F] fp16/bf16 intermediates) with 32-bit per-lane BYTE
  // offsets, so each such matrix must hold fewer than 2^31 elements.
  constexpr int64_t LIM = (int64_t)1 << 31;
  if ((int64_t)sh->T * sh->d >= LIM || (int64_t)sh->F * sh->d >= LIM || (int64_t)sh->T * sh->F >= LIM)
    return fail(TWELL_EUNSUPPORTED, "T*d, F*d and T*F must each be below 2^31 (T=%d d=%d F=%d)", sh->T, sh->d,
                sh->F);
  return TWELL_OK;
}

twell_status check_mat(const twell_mat* m, bool need_mask) {
  if (!m) return fail(TWELL_EINVAL, "twell_mat is NULL");
  if (m->T < 0 || m->F <= 0) return fail(TWELL_EINVAL, "bad twell_mat shape T=%d F=%d", m->T, m->F);
  if (m->R != GPU_R || m->C != GPU_C)
    return fail(TWELL_EUNSUPPORTED, "GPU TwELL tiles are 16 x 64 (got %d x %d)", m->R, m->C);
  if (m->F % GPU_C != 0) return fail(TWELL_EUNSUPPORTED, "F=%d is not a multiple of 64", m->F);
  if (m->vdtype != TWELL_F32 && m->vdtype != TWELL_BF16) return fail(TWELL_EINVAL, "bad value dtype");
  if (m->T > 0 && (!m->cnt || !m->width || !m->val || !m->idx))
    return fail(TWELL_EINVAL, "twell_mat array is NULL");
  if (need_mask && m->T > 0 && !m->mask) return fail(TWELL_EINVAL, "twell_mat mask is required here");
  if (!aligned16(m->val) || !aligned16(m->mask)) return fail(TWELL_EINVAL, "twell_mat arrays must be 16-byte aligned");
  return TWELL_OK;
}

void cmat_parts(int64_t T, int64_t F, int64_t W, size_t parts[6]) {
  const int64_t NR = (T + GPU_R - 1) / GPU_R, NT = F / GPU_C;
  parts[0] = (size_t)(T * NT);
  parts[1] = (size_t)(NR * NT);
  parts[2] = (size_t)(NR * NT * W * GPU_R) * 4;
  parts[3] = (size_t)(NR * NT * W * GPU_R);
  parts[4] = (size_t)(T * NT) * 8;
  parts[5] = (size_t)T;
}

twell_status check_cmat(const twell_cmat* m) {
  if (!m) return fail(TWELL_EINVAL, "twell_cmat is NULL");
  if (m->T < 0 || m->F <= 0) return fail(TWELL_EINVAL, "bad twell_cmat shape T=%d F=%d", m->T, m->F);
  if (m->F % GPU_C != 0) return fail(TWELL_EUNSUPPORTED, "F=%d is not a multiple of 64", m->F);
  if (m->W < 1 || m->W > GPU_C) return fail(TWELL_EINVAL, "capacity W=%d outside 1..64", m->W);
  if (m->T > 0 && (!m->cnt || !m->width || !m->val || !m->idx || !m->mask || !m->ovf))
    return fail(TWELL_EINVAL, "twell_cmat array is NULL");
  if (!aligned16(m->val) || !aligned16(m->mask)) return fail(TWELL_EINVAL, "twell_cmat arrays must be 16-byte aligned");
  return TWELL_OK;
}

TwellView view_of(const twell_mat* m) {
  TwellView v;
  v.T = m->T; v.F = m->F; v.NT = m->F / GPU_C; v.NR = (m->T + GPU_R - 1) / GPU_R;
  v.cnt = m->cnt; v.width = m->width; v.val = m->val; v.idx = m->idx; v.mask = m->mask;
  return v;
}

// The compact form read in place: the same arrays with W slots per tile.
TwellView view_of(const twell_cmat* m) {
  TwellView v;
  v.T = m->T; v.F = m->F; v.NT = m->F / GPU_C; v.NR = (m->T + GPU_R - 1) / GPU_R;
  v.cnt = m->cnt; v.width = m->width; v.val = m->val; v.idx = m->idx; v.mask = m->mask;
  v.cap = m->W;
  return v;
}

// Workspace of the forward: one TwELL (fp32 values, with mask; with saved_h
// only its value array is used, for a); training adds the row classification
// and the dense rows' activation buffer.
struct FwdWs {
  TwellView h;
  uint8_t* flag;
  int* list;
  int* nD;
  float* act;
  void* uni;         // union-GEMM workspace (bf16 inputs)
  void* dec;         // few-token path workspace (bf16 inference, T <= DECODE_T_MAX)
};

bool few_token_path(const twell_ffn_shape* sh, bool training) {
  return sh->in_dt == TWELL_BF16 && !training && sh->T > 0 && sh->T <= DECODE_T_MAX;
}

size_t fwd_layout(const twell_ffn_shape* sh, bool training, void* ws, FwdWs* out) {
  size_t parts[5];
  mat_parts(sh->T, sh->F, GPU_R, GPU_C, TWELL_F32, parts);
  Carver c(ws);
  FwdWs w{};
  if (training) {
    w.flag = (uint8_t*)c.take((size_t)sh->T);
    w.list = (int*)c.take((size_t)sh->T * 4);
    w.nD = (int*)c.take(4);
  }
  // the dense rows' activation buffer overlays the sparse phases' buffers:
  // the dense-row forward runs after the down-projection, on the same stream
  size_t act_end = 0;
  if (training) {
    Carver dn(ws ? (char*)ws + c.off : nullptr);
    w.act = (float*)dn.take((size_t)dense_row_cap(sh->T) * sh->F * 4);   // one round of dense rows
    act_end = c.off + dn.off;
  }
  TwellView& v = w.h;
  v.T = sh->T; v.F = sh->F; v.NT = sh->F / GPU_C; v.NR = (sh->T + GPU_R - 1) / GPU_R;
  v.cnt = (uint8_t*)c.take(parts[0]);
  v.width = (uint8_t*)c.take(parts[1]);
  v.val = c.take(parts[2]);
  v.idx = (uint8_t*)c.take(parts[3]);
  v.mask = (uint64_t*)c.take(parts[4]);
  if (few_token_path(sh, training)) {
    w.dec = c.take(decode_ws_bytes(sh->T, sh->d, sh->F));
  } else if (sh->in_dt == TWELL_BF16) {
    w.uni = c.take(union_ws_bytes(sh->T, sh->d, sh->F));
  }
  if (out) *out = w;
  return c.off > act_end ? c.off : act_end;
}

// Workspace of the capacity-bounded forward (T > DECODE_T_MAX): the TwELL of
// h with W slots per tile, then the union workspace whose a rows hold ucap
// positions.  Few-token shapes take the ordinary inference layout.
bool bounded_caps_ok(const twell_ffn_shape* sh, int32_t W, int32_t ucap) {
  return W >= 4 && W <= GPU_C && W % 4 == 0 && ucap >= 64 && ucap <= sh->F && ucap % 64 == 0;
}

size_t bounded_layout(const twell_ffn_shape* sh, int32_t W, int32_t ucap, void* ws, FwdWs* out) {
  if (few_token_path(sh, false)) return fwd_layout(sh, false, ws, out);
  size_t parts[6];
  cmat_parts(sh->T, sh->F, W, parts);
  Carver c(ws);
  FwdWs w{};
  TwellView& v = w.h;
  v.T = sh->T; v.F = sh->F; v.NT = sh->F / GPU_C; v.NR = (sh->T + GPU_R - 1) / GPU_R;
  v.cap = W;
  v.cnt = (uint8_t*)c.take(parts[0]);
  v.width = (uint8_t*)c.take(parts[1]);
  v.val = c.take(parts[2]);
  v.idx = (uint8_t*)c.take(parts[3]);
  v.mask = (uint64_t*)c.take(parts[4]);
  w.uni = c.take(union_ws_bytes(sh->T, sh->d, sh->F, ucap));
  if (out) *out = w;
  return c.off;
}

// Workspace of the hybrid backward.
struct BwdWs {
  uint8_t* flag;
  int* list;
  int* nD;
  float* buf3;       // [T][3F]
  float* dbg_part;   // [ceil(T/64)][F]
  float* aval;       // TwELL-shaped value arrays
  float* dgval;
  float* duval;
  int* part;         // [ceil(T/256)][F]
  int* start;        // [F+1]
  uint32_t* entries; // one per stored pair of a sparse row
  void* uni;         // bf16 inputs: union lists of the sparse rows
};

size_t bwd_layout(const twell_ffn_shape* sh, int32_t tau, void* ws, BwdWs* out, int cap = GPU_C) {
  const int64_t T = sh->T, F = sh->F;
  const int64_t NR = (T + GPU_R - 1) / GPU_R, NT = F / GPU_C;
  const size_t slots = (size_t)(NR * NT * cap * GPU_R);   // the value arrays follow h's capacity
  // a sparse row holds at most min(F, tau) pairs
  const int64_t per_row = tau < 0 ? 0 : (tau < F ? tau : F);
  Carver c(ws);
  BwdWs w{};
  w.flag = (uint8_t*)c.take((size_t)T);
  w.list = (int*)c.take((size_t)T * 4);
  w.nD = (int*)c.take(4);
  // the dense-row branch runs to its end before the sparse branch starts (one
  // stream), so the sparse branch's buffers overlay the dense branch's
  Carver dn(ws ? (char*)ws + c.off : nullptr);
  dn.off = 0;
  // the dense rows go in rounds of dense_row_cap(T) rows
  const int64_t DC = dense_row_cap((int)T);
  w.buf3 = (float*)dn.take((size_t)(DC * 3 * F) * 4);
  w.dbg_part = (float*)dn.take((size_t)(((DC + 63) / 64) * F) * 4);
  const size_t dense_end = c.off + dn.off;
  w.aval = (float*)c.take(slots * 4);
  w.dgval = (float*)c.take(slots * 4);
  w.duval = (float*)c.take(slots * 4);
  w.part = (int*)c.take((size_t)(((T + 255) / 256) * F) * 4);
  w.start = (int*)c.take((size_t)(F + 1) * 4);
  w.entries = (uint32_t*)c.take((size_t)(T * per_row) * 4);
  if (sh->in_dt == TWELL_BF16) w.uni = c.take(union_bwd_ws_bytes((int)T, sh->d, (int)F));
  if (out) *out = w;
  return c.off > dense_end ? c.off : dense_end;
}

}  // namespace

extern "C" {

size_t twell_mat_bytes(int32_t T, int32_t F, int32_t R, int32_t C, twell_dtype vdtype, size_t parts[5]) {
  size_t p[5] = {0, 0, 0, 0, 0};
  if (T >= 0 && F > 0 && R > 0 && C > 0) mat_parts(T, F, R, C, vdtype, p);
  if (parts) memcpy(parts, p, sizeof(p));
  return p[0] + p[1] + p[2] + p[3] + p[4];
}

twell_status twell_pack(const void* G, twell_dtype gdtype, int64_t ldg, twell_mat* out, hipStream_t stream) {
  twell_status st = check_mat(out, false);
  if (st) return st;
  if (gdtype != out->vdtype) return fail(TWELL_EINVAL, "twell_pack stores bit copies: vdtype must equal the dtype of G");
  if (ldg < out->F) return fail(TWELL_EINVAL, "ldg=%lld < F=%d", (long long)ldg, out->F);
  if (out->T == 0) return TWELL_OK;
  if (!G) return fail(TWELL_EINVAL, "G is NULL");
  return hip_status(launch_pack(G, gdtype == TWELL_BF16 ? DT_BF16 : DT_F32, ldg, view_of(out), stream), "twell_pack");
}

twell_status twell_unpack(const twell_mat* in, void* H, int64_t ldh, hipStream_t stream) {
  twell_status st = check_mat(in, false);
  if (st) return st;
  if (ldh < in->F) return fail(TWELL_EINVAL, "ldh=%lld < F=%d", (long long)ldh, in->F);
  if (in->T == 0) return TWELL_OK;
  if (!H) return fail(TWELL_EINVAL, "H is NULL");
  return hip_status(launch_unpack(view_of(in), in->vdtype == TWELL_BF16 ? DT_BF16 : DT_F32, H, ldh, stream),
                    "twell_unpack");
}

size_t twell_ffn_fwd_workspace(const twell_ffn_shape* sh, int32_t training) {
  if (!sh || check_shape(sh) != TWELL_OK) return 0;
  // a workspace sized for training also serves an inference call of the same shape
  const size_t inf = fwd_layout(sh, false, nullptr, nullptr);
  if (!training) return inf;
  const size_t tr = fwd_layout(sh, true, nullptr, nullptr);
  return tr > inf ? tr : inf;
}

twell_status twell_ffn_fwd_ex(const twell_ffn_shape* sh, const void* x, const void* WgT, const void* bg,
                              const void* WuT, const void* Wd, void* y, twell_mat* saved_h,
                              int32_t dense_row_threshold, void* ws, size_t ws_bytes, hipStream_t stream,
                              hipEvent_t* stage_events, int32_t n_events) {
  twell_status st = check_shape(sh);
  if (st) return st;
  if (sh->T > 0 && (!x || !WgT || !WuT || !Wd || !y)) return fail(TWELL_EINVAL, "NULL tensor argument");
  if (!aligned16(x) || !aligned16(WgT) || !aligned16(WuT) || !aligned16(Wd) || !aligned16(y) || !aligned16(bg))
    return fail(TWELL_EINVAL, "tensors must be 16-byte aligned");
  if (saved_h) {
    st = check_mat(saved_h, true);
    if (st) return st;
    if (saved_h->T != sh->T || saved_h->F != sh->F || saved_h->vdtype != TWELL_F32)
      return fail(TWELL_EINVAL, "saved_h must be T x F with fp32 values");
  }
  if (n_events < 0 || (n_events > 0 && !stage_events)) return fail(TWELL_EINVAL, "bad stage event array");
  const bool training = dense_row_threshold >= 0;
  if (training && !saved_h) return fail(TWELL_EINVAL, "the hybrid forward (dense_row_threshold >= 0) needs saved_h");
  const size_t need = fwd_layout(sh, training, nullptr, nullptr);
  if (!ws || ws_bytes < need) return fail(TWELL_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (sh->T == 0) return TWELL_OK;

  FwdWs w;
  fwd_layout(sh, training, ws, &w);
  const int in_dt = sh->in_dt == TWELL_BF16 ? DT_BF16 : DT_F32;
  const int out_dt = sh->out_dt == TWELL_BF16 ? DT_BF16 : DT_F32;
  TwellView h = w.h;
  float* aval = (float*)w.h.val;             // a overwrites h in place
  if (saved_h) {
    h = view_of(saved_h);                    // h is kept for the backward pass
    aval = (float*)w.h.val;
  }
  auto evt = [&](int i) -> hipEvent_t { return i < n_events ? stage_events[i] : nullptr; };
  auto mark = [&](int i) {
    if (i < n_events) (void)hipEventRecord(stage_events[i], stream);
  };
  mark(0);                                                            // start
  if (few_token_path(sh, training)) {
    hipError_t e = launch_decode_fwd(x, WgT, bg, WuT, Wd, sh->T, sh->d, sh->F, h, w.dec, y, out_dt, stream,
                                     evt(1), evt(2), evt(3));
    if (e != hipSuccess) return hip_status(e, "few-token forward");
    mark(4);
    mark(5);
    mark(6);
    return TWELL_OK;
  }
  // inference with bf16 inputs: the gate epilogue also writes the slab unions
  // the up/down GEMMs' lists are built from (and clears their overflow flag)
  const bool slabs_ready = !training && in_dt == DT_BF16;
  uint64_t* slabs = nullptr;
  int* uflag = nullptr;
  if (slabs_ready) union_slabs_and_flag(sh->T, sh->F, w.uni, &slabs, &uflag);
  hipError_t e = launch_gate_twell(in_dt, x, WgT, bg, sh->T, sh->d, sh->F, h, stream, slabs, uflag);
  if (e != hipSuccess) return hip_status(e, "gate GEMM");
  const uint8_t* skip = nullptr;
  if (training) {
    e = launch_classify(h, dense_row_threshold, w.flag, w.list, w.nD, nullptr, stream);
    if (e != hipSuccess) return hip_status(e, "row classification");
    skip = w.flag;
  }
  mark(1);                                                            // gate GEMM + pack done
  if (in_dt == DT_BF16) {
    // a value beyond the fp16 range sets the overflow flag, and the down kernel
    // then computes y per stored pair in fp32 instead (no extra launch)
    e = launch_union_fwd(x, WuT, Wd, sh->T, sh->d, sh->F, h, skip, w.uni, y, out_dt, nullptr, stream, evt(2), evt(3),
                         slabs_ready);
    if (e != hipSuccess) return hip_status(e, "union up/down GEMMs");
    mark(4);                                                          // down-projection done
  } else {
    mark(2);
    e = launch_sddmm_up(in_dt, x, WuT, sh->T, sh->d, sh->F, h, aval, skip, stream);
    if (e != hipSuccess) return hip_status(e, "sparse up-projection");
    mark(3);
    e = launch_spmm_down(in_dt, out_dt, aval, Wd, sh->T, sh->d, sh->F, h, y, skip, stream);
    if (e != hipSuccess) return hip_status(e, "sparse down-projection");
    mark(4);
  }
  mark(5);                                                            // sparse phases done
  if (training) {
    e = launch_dense_rows_fwd(in_dt, x, WgT, bg, WuT, Wd, sh->T, sh->d, sh->F, w.list, w.nD, w.act, out_dt, y,
                              stream);
    if (e != hipSuccess) return hip_status(e, "dense-row forward");
  }
  mark(6);                                                            // end
  return TWELL_OK;
}

twell_status twell_ffn_fwd(const twell_ffn_shape* sh, const void* x, const void* WgT, const void* bg,
                           const void* WuT, const void* Wd, void* y, twell_mat* saved_h,
                           int32_t dense_row_threshold, void* ws, size_t ws_bytes, hipStream_t stream) {
  return twell_ffn_fwd_ex(sh, x, WgT, bg, WuT, Wd, y, saved_h, dense_row_threshold, ws, ws_bytes, stream, nullptr, 0);
}

size_t twell_ffn_fwd_bounded_workspace(const twell_ffn_shape* sh, int32_t tile_cap, int32_t union_cap) {
  if (!sh || check_shape(sh) != TWELL_OK || sh->in_dt != TWELL_BF16 || !bounded_caps_ok(sh, tile_cap, union_cap))
    return 0;
  return bounded_layout(sh, tile_cap, union_cap, nullptr, nullptr);
}

twell_status twell_ffn_fwd_bounded(const twell_ffn_shape* sh, const void* x, const void* WgT, const void* bg,
                                   const void* WuT, const void* Wd, void* y, int32_t tile_cap, int32_t union_cap,
                                   int32_t* n_over_blocks, void* ws, size_t ws_bytes, hipStream_t stream) {
  twell_status st = check_shape(sh);
  if (st) return st;
  if (sh->in_dt != TWELL_BF16) return fail(TWELL_EUNSUPPORTED, "the bounded forward takes bf16 inputs");
  if (!bounded_caps_ok(sh, tile_cap, union_cap))
    return fail(TWELL_EINVAL, "tile_cap=%d must be a multiple of 4 in 4..64 and union_cap=%d a multiple of 64 in "
                "64..F=%d", tile_cap, union_cap, sh->F);
  if (sh->T > 0 && (!x || !WgT || !WuT || !Wd || !y)) return fail(TWELL_EINVAL, "NULL tensor argument");
  if (!aligned16(x) || !aligned16(WgT) || !aligned16(WuT) || !aligned16(Wd) || !aligned16(y) || !aligned16(bg))
    return fail(TWELL_EINVAL, "tensors must be 16-byte aligned");
  const size_t need = bounded_layout(sh, tile_cap, union_cap, nullptr, nullptr);
  if (!ws || ws_bytes < need) return fail(TWELL_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (few_token_path(sh, false) || sh->T == 0) {
    st = twell_ffn_fwd_ex(sh, x, WgT, bg, WuT, Wd, y, nullptr, -1, ws, ws_bytes, stream, nullptr, 0);
    if (st || !n_over_blocks) return st;
    return hip_status(launch_union_over_count(0, sh->F, nullptr, 0, n_over_blocks, stream), "block count");
  }
  FwdWs w;
  bounded_layout(sh, tile_cap, union_cap, ws, &w);
  const int out_dt = sh->out_dt == TWELL_BF16 ? DT_BF16 : DT_F32;
  uint64_t* slabs = nullptr;
  int* uflag = nullptr;
  union_slabs_and_flag(sh->T, sh->F, w.uni, &slabs, &uflag);
  hipError_t e = launch_gate_twell(DT_BF16, x, WgT, bg, sh->T, sh->d, sh->F, w.h, stream, slabs, uflag);
  if (e != hipSuccess) return hip_status(e, "gate GEMM");
  e = launch_union_fwd(x, WuT, Wd, sh->T, sh->d, sh->F, w.h, nullptr, w.uni, y, out_dt, nullptr, stream, nullptr,
                       nullptr, true, WgT, bg, union_cap);
  if (e != hipSuccess) return hip_status(e, "union up/down GEMMs");
  if (n_over_blocks) e = launch_union_over_count(sh->T, sh->F, w.uni, union_cap, n_over_blocks, stream);
  return hip_status(e, "block count");
}

size_t twell_ffn_bwd_workspace(const twell_ffn_shape* sh, int32_t dense_row_threshold) {
  if (!sh || check_shape(sh) != TWELL_OK) return 0;
  return bwd_layout(sh, dense_row_threshold, nullptr, nullptr);
}

static twell_status bwd_run(const twell_ffn_shape* sh, const void* x, const void* WgT, const void* bg,
                            const void* WuT, const void* Wd, const void* dY, const TwellView& h,
                            const uint8_t* force, int32_t dense_row_threshold, float l1_lambda,
                            int32_t l1_per_token_mean, float* dX, float* dWgT, float* dWuT, float* dWd, float* dbg,
                            int32_t* n_dense_rows, const BwdWs& w, hipStream_t stream);

// Checks shared by the hybrid backward entry points (all but the saved state).
static twell_status check_bwd_args(const twell_ffn_shape* sh, const void* x, const void* WgT, const void* bg,
                                   const void* WuT, const void* Wd, const void* dY, float l1_lambda,
                                   int32_t l1_per_token_mean, float* dX, float* dWgT, float* dWuT, float* dWd,
                                   float* dbg) {
  twell_status st = check_shape(sh);
  if (!(l1_lambda >= 0.f) || l1_lambda > 3.0e38f)
    return fail(TWELL_EINVAL, "l1_lambda must be finite and >= 0 (got %g)", (double)l1_lambda);
  if (l1_per_token_mean != 0 && l1_per_token_mean != 1)
    return fail(TWELL_EINVAL, "l1_per_token_mean must be 0 or 1");
  if (st) return st;
  if (!WgT || !WuT || !Wd || !dWgT || !dWuT || !dWd) return fail(TWELL_EINVAL, "NULL weight or gradient argument");
  if (sh->T > 0 && (!x || !dY || !dX)) return fail(TWELL_EINVAL, "NULL tensor argument");
  for (const void* p : {x, WgT, bg, WuT, Wd, dY, (const void*)dX, (const void*)dWgT, (const void*)dWuT,
                        (const void*)dWd, (const void*)dbg})
    if (!aligned16(p)) return fail(TWELL_EINVAL, "tensors must be 16-byte aligned");
  const int64_t NR = (sh->T + GPU_R - 1) / GPU_R;
  if (NR * (sh->F / GPU_C) * GPU_C * GPU_R >= ((int64_t)1 << 32))
    return fail(TWELL_EUNSUPPORTED, "T x F too large for 32-bit TwELL slot offsets");
  // the dense branch's [rows][3F] fp32 buffer is read with 32-bit element offsets
  if ((int64_t)sh->T * 3 * sh->F >= ((int64_t)1 << 32))
    return fail(TWELL_EUNSUPPORTED, "3*T*F must be below 2^32 for the backward (T=%d F=%d)", sh->T, sh->F);
  return TWELL_OK;
}

twell_status twell_ffn_bwd_hybrid(const twell_ffn_shape* sh, const void* x, const void* WgT, const void* bg,
                                  const void* WuT, const void* Wd, const void* dY, const twell_mat* saved_h,
                                  int32_t dense_row_threshold, float* dX, float* dWgT, float* dWuT, float* dWd,
                                  float* dbg, int32_t* n_dense_rows, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  return twell_ffn_bwd_hybrid_l1(sh, x, WgT, bg, WuT, Wd, dY, saved_h, dense_row_threshold, 0.f, 0, dX, dWgT, dWuT,
                                 dWd, dbg, n_dense_rows, ws, ws_bytes, stream);
}

twell_status twell_ffn_bwd_hybrid_l1(const twell_ffn_shape* sh, const void* x, const void* WgT, const void* bg,
                                     const void* WuT, const void* Wd, const void* dY, const twell_mat* saved_h,
                                     int32_t dense_row_threshold, float l1_lambda, int32_t l1_per_token_mean,
                                     float* dX, float* dWgT, float* dWuT, float* dWd, float* dbg,
                                     int32_t* n_dense_rows, void* ws, size_t ws_bytes, hipStream_t stream) {
  twell_status st = check_bwd_args(sh, x, WgT, bg, WuT, Wd, dY, l1_lambda, l1_per_token_mean, dX, dWgT, dWuT, dWd,
                                   dbg);
  if (st) return st;
  st = check_mat(saved_h, true);
  if (st) return st;
  if (saved_h->T != sh->T || saved_h->F != sh->F || saved_h->vdtype != TWELL_F32)
    return fail(TWELL_EINVAL, "saved_h must be T x F with fp32 values");
  const size_t need = bwd_layout(sh, dense_row_threshold, nullptr, nullptr);
  if (!ws || ws_bytes < need) return fail(TWELL_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);

  BwdWs w;
  bwd_layout(sh, dense_row_threshold, ws, &w);
  return bwd_run(sh, x, WgT, bg, WuT, Wd, dY, view_of(saved_h), nullptr, dense_row_threshold, l1_lambda,
                 l1_per_token_mean, dX, dWgT, dWuT, dWd, dbg, n_dense_rows, w, stream);
}

// Both hybrid backward entry points after their checks: h is the capacity-64
// TwELL of the forward's activations; rows with force[t] set (may be null)
// take the dense branch whatever their count.
static twell_status bwd_run(const twell_ffn_shape* sh, const void* x, const void* WgT, const void* bg,
                            const void* WuT, const void* Wd, const void* dY, const TwellView& h,
                            const uint8_t* force, int32_t dense_row_threshold, float l1_lambda,
                            int32_t l1_per_token_mean, float* dX, float* dWgT, float* dWuT, float* dWd, float* dbg,
                            int32_t* n_dense_rows, const BwdWs& w, hipStream_t stream) {
  const int in_dt = sh->in_dt == TWELL_BF16 ? DT_BF16 : DT_F32;
  const int T = sh->T, d = sh->d, F = sh->F;
  // gradient coefficient of the penalty: lambda for a sum over the
  // activations, lambda / T for a mean over tokens
  const float l1 = (l1_per_token_mean && T > 0) ? l1_lambda / (float)T : l1_lambda;
  hipError_t e = launch_classify(h, dense_row_threshold, w.flag, w.list, w.nD, n_dense_rows, stream, force);
  if (e != hipSuccess) return hip_status(e, "row classification");
  e = launch_dense_rows_bwd(in_dt, x, WgT, bg, WuT, Wd, dY, T, d, F, w.list, w.nD, w.buf3, w.dbg_part, dX, dWgT,
                            dWuT, dWd, dbg, stream, l1);
  if (e != hipSuccess) return hip_status(e, "dense-row backward");
  if (in_dt == DT_BF16) {
    int* ovf = nullptr;
    e = launch_union_bwd(x, dY, WgT, WuT, Wd, T, d, F, h, w.flag, w.uni, w.aval, w.dgval, w.duval, l1, dX, &ovf,
                         stream);
    if (e != hipSuccess) return hip_status(e, "sparse backward union GEMMs");
    // a value beyond the fp16 range: dX of the sparse rows per pair in fp32 (does nothing unless the flag is set)
    e = launch_down_bf16(w.dgval, w.duval, WgT, WuT, T, d, F, h, dX, DT_F32, w.flag, stream, ovf);
    if (e != hipSuccess) return hip_status(e, "sparse backward dX fallback");
  } else {
    e = launch_sddmm_bwd(in_dt, x, dY, WuT, Wd, T, d, F, h, w.aval, w.dgval, w.duval, w.flag, stream, l1);
    if (e != hipSuccess) return hip_status(e, "sparse backward SDDMM");
    e = launch_spmm_dx(in_dt, w.dgval, w.duval, WgT, WuT, T, d, F, h, dX, w.flag, stream);
    if (e != hipSuccess) return hip_status(e, "sparse backward dX");
  }
  e = launch_sparse_wgrad(in_dt, x, dY, T, d, F, h, w.flag, w.part, w.start, w.entries, w.aval, w.dgval,
                          w.duval, dWgT, dWuT, dWd, dbg, stream);
  return hip_status(e, "sparse weight gradients");
}

// ------------------------------------------------------------------ compact TwELL

size_t twell_cmat_bytes(int32_t T, int32_t F, int32_t W, size_t parts[6]) {
  size_t p[6] = {0, 0, 0, 0, 0, 0};
  if (T >= 0 && F > 0 && F % GPU_C == 0 && W >= 1 && W <= GPU_C) cmat_parts(T, F, W, p);
  if (parts) memcpy(parts, p, sizeof(p));
  return p[0] + p[1] + p[2] + p[3] + p[4] + p[5];
}

static CompactArgs compact_args(const twell_mat* full, const twell_cmat* c) {
  CompactArgs a{};
  a.T = c->T; a.NT = c->F / GPU_C; a.W = c->W;
  a.ntiles = (int64_t)((c->T + GPU_R - 1) / GPU_R) * a.NT;
  if (full) {   // null: the compact arrays alone (after a gate GEMM packed into them)
    a.cnt = full->cnt; a.width = full->width; a.val = (float*)full->val; a.idx = full->idx; a.mask = full->mask;
  }
  a.ccnt = c->cnt; a.cwidth = c->width; a.cval = c->val; a.cidx = c->idx; a.cmask = c->mask; a.ovf = c->ovf;
  return a;
}

static twell_status check_pair(const twell_mat* full, const twell_cmat* c) {
  twell_status st = check_mat(full, true);
  if (st) return st;
  st = check_cmat(c);
  if (st) return st;
  if (full->vdtype != TWELL_F32) return fail(TWELL_EINVAL, "compact TwELL holds fp32 values");
  if (full->T != c->T || full->F != c->F)
    return fail(TWELL_EINVAL, "shape mismatch: %d x %d vs %d x %d", full->T, full->F, c->T, c->F);
  return TWELL_OK;
}

twell_status twell_compact(const twell_mat* full, twell_cmat* out, hipStream_t stream) {
  twell_status st = check_pair(full, out);
  if (st) return st;
  if (out->T == 0) return TWELL_OK;
  return hip_status(launch_compact(compact_args(full, out), false, stream), "twell_compact");
}

twell_status twell_expand(const twell_cmat* in, twell_mat* full, hipStream_t stream) {
  twell_status st = check_pair(full, in);
  if (st) return st;
  if (in->T == 0) return TWELL_OK;
  return hip_status(launch_compact(compact_args(full, in), true, stream), "twell_expand");
}

// The compact backward's workspace: the hybrid backward's, then a
// capacity-64 value and index array that the stored slots are moved into.
size_t twell_ffn_bwd_compact_workspace(const twell_ffn_shape* sh, int32_t dense_row_threshold, int32_t W) {
  if (!sh || check_shape(sh) != TWELL_OK || W < 1 || W > GPU_C) return 0;
  return bwd_layout(sh, dense_row_threshold, nullptr, nullptr, W);
}

twell_status twell_ffn_bwd_hybrid_compact(const twell_ffn_shape* sh, const void* x, const void* WgT,
                                          const void* bg, const void* WuT, const void* Wd, const void* dY,
                                          const twell_cmat* saved, int32_t dense_row_threshold, float l1_lambda,
                                          int32_t l1_per_token_mean, float* dX, float* dWgT, float* dWuT,
                                          float* dWd, float* dbg, int32_t* n_dense_rows, void* ws,
                                          size_t ws_bytes, hipStream_t stream) {
  twell_status st = check_bwd_args(sh, x, WgT, bg, WuT, Wd, dY, l1_lambda, l1_per_token_mean, dX, dWgT, dWuT, dWd,
                                   dbg);
  if (st) return st;
  st = check_cmat(saved);
  if (st) return st;
  if (saved->T != sh->T || saved->F != sh->F)
    return fail(TWELL_EINVAL, "saved must be T x F (T=%d F=%d)", sh->T, sh->F);
  const size_t need = bwd_layout(sh, dense_row_threshold, nullptr, nullptr, saved->W);
  if (!ws || ws_bytes < need) return fail(TWELL_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  BwdWs w;
  bwd_layout(sh, dense_row_threshold, ws, &w, saved->W);
  // the compact arrays are read in place (W slots per tile); the per-pair
  // values of the backward follow the same layout
  return bwd_run(sh, x, WgT, bg, WuT, Wd, dY, view_of(saved), saved->ovf, dense_row_threshold, l1_lambda,
                 l1_per_token_mean, dX, dWgT, dWuT, dWd, dbg, n_dense_rows, w, stream);
}

// Workspace of the compact training forward: the row classification, the
// dense rows' activation buffer, a at the stored pairs (capacity W; fp32
// inputs) and the union workspace (bf16 inputs).
static size_t fwd_compact_layout(const twell_ffn_shape* sh, int32_t W, void* ws, FwdWs* out, float** aval) {
  Carver c(ws);
  FwdWs w{};
  w.flag = (uint8_t*)c.take((size_t)sh->T);
  w.list = (int*)c.take((size_t)sh->T * 4);
  w.nD = (int*)c.take(4);
  // the dense rows' activation buffer overlays the sparse phases' buffers
  // (the dense-row forward runs after the down-projection, on the same stream)
  Carver dn(ws ? (char*)ws + c.off : nullptr);
  w.act = (float*)dn.take((size_t)dense_row_cap(sh->T) * sh->F * 4);    // one round of dense rows
  const size_t act_end = c.off + dn.off;
  float* av = nullptr;
  if (sh->in_dt == TWELL_BF16) {
    w.uni = c.take(union_ws_bytes(sh->T, sh->d, sh->F));
  } else {
    size_t parts[6];
    cmat_parts(sh->T, sh->F, W, parts);
    av = (float*)c.take(parts[2]);
  }
  if (out) *out = w;
  if (aval) *aval = av;
  return c.off > act_end ? c.off : act_end;
}

size_t twell_ffn_fwd_compact_workspace(const twell_ffn_shape* sh, int32_t W) {
  if (!sh || check_shape(sh) != TWELL_OK || W < 1 || W > GPU_C) return 0;
  return fwd_compact_layout(sh, W, nullptr, nullptr, nullptr);
}

twell_status twell_ffn_fwd_compact(const twell_ffn_shape* sh, const void* x, const void* WgT, const void* bg,
                                   const void* WuT, const void* Wd, void* y, twell_cmat* saved,
                                   int32_t dense_row_threshold, void* ws, size_t ws_bytes, hipStream_t stream) {
  twell_status st = check_shape(sh);
  if (st) return st;
  if (sh->T > 0 && (!x || !WgT || !WuT || !Wd || !y)) return fail(TWELL_EINVAL, "NULL tensor argument");
  if (!aligned16(x) || !aligned16(WgT) || !aligned16(WuT) || !aligned16(Wd) || !aligned16(y) || !aligned16(bg))
    return fail(TWELL_EINVAL, "tensors must be 16-byte aligned");
  st = check_cmat(saved);
  if (st) return st;
  if (saved->T != sh->T || saved->F != sh->F)
    return fail(TWELL_EINVAL, "saved must be T x F (T=%d F=%d)", sh->T, sh->F);
  if (dense_row_threshold < 0) return fail(TWELL_EINVAL, "the compact forward is the hybrid one: threshold >= 0");
  const size_t need = fwd_compact_layout(sh, saved->W, nullptr, nullptr, nullptr);
  if (!ws || ws_bytes < need) return fail(TWELL_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (sh->T == 0) return TWELL_OK;
  FwdWs w;
  float* aval = nullptr;
  fwd_compact_layout(sh, saved->W, ws, &w, &aval);
  const int in_dt = sh->in_dt == TWELL_BF16 ? DT_BF16 : DT_F32;
  const int out_dt = sh->out_dt == TWELL_BF16 ? DT_BF16 : DT_F32;
  const TwellView h = view_of(saved);
  // the gate epilogue packs straight into the W slots of each tile; then the
  // rows with a tile above W are flagged, widths clamped, and those rows go
  // to the dense branch with the rows above the threshold
  hipError_t e = launch_gate_twell(in_dt, x, WgT, bg, sh->T, sh->d, sh->F, h, stream);
  if (e != hipSuccess) return hip_status(e, "gate GEMM");
  e = launch_compact_finish(compact_args(nullptr, saved), stream);
  if (e != hipSuccess) return hip_status(e, "compact overflow flags");
  e = launch_classify(h, dense_row_threshold, w.flag, w.list, w.nD, nullptr, stream, saved->ovf);
  if (e != hipSuccess) return hip_status(e, "row classification");
  if (in_dt == DT_BF16) {
    e = launch_union_fwd(x, WuT, Wd, sh->T, sh->d, sh->F, h, w.flag, w.uni, y, out_dt, nullptr, stream);
    if (e != hipSuccess) return hip_status(e, "union up/down GEMMs");
  } else {
    e = launch_sddmm_up(in_dt, x, WuT, sh->T, sh->d, sh->F, h, aval, w.flag, stream);
    if (e != hipSuccess) return hip_status(e, "sparse up-projection");
    TwellView pat = h;
    e = launch_spmm_down(in_dt, out_dt, aval, Wd, sh->T, sh->d, sh->F, pat, y, w.flag, stream);
    if (e != hipSuccess) return hip_status(e, "sparse down-projection");
  }
  e = launch_dense_rows_fwd(in_dt, x, WgT, bg, WuT, Wd, sh->T, sh->d, sh->F, w.list, w.nD, w.act, out_dt, y, stream);
  return hip_status(e, "dense-row forward");
}

static twell_status check_tensors(const twell_ffn_shape* sh, std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs) {
    if (sh->T > 0 && !p) return fail(TWELL_EINVAL, "NULL tensor argument");
    if (!aligned16(p)) return fail(TWELL_EINVAL, "tensors must be 16-byte aligned");
  }
  return TWELL_OK;
}

static twell_status check_h(const twell_ffn_shape* sh, const twell_mat* h) {
  twell_status st = check_mat(h, true);
  if (st) return st;
  if (h->T != sh->T || h->F != sh->F || h->vdtype != TWELL_F32)
    return fail(TWELL_EINVAL, "TwELL matrix must be T x F (T=%d F=%d) with fp32 values", sh->T, sh->F);
  return TWELL_OK;
}

twell_status twell_gate_pack(const twell_ffn_shape* sh, const void* x, const void* WgT, const void* bg,
                             twell_mat* h, hipStream_t stream) {
  twell_status st = check_shape(sh);
  if (!st) st = check_tensors(sh, {x, WgT});
  if (!st && !aligned16(bg)) st = fail(TWELL_EINVAL, "bg must be 16-byte aligned");
  if (!st) st = check_h(sh, h);
  if (st) return st;
  if (sh->T == 0) return TWELL_OK;
  return hip_status(launch_gate_twell(sh->in_dt == TWELL_BF16 ? DT_BF16 : DT_F32, x, WgT, bg, sh->T, sh->d,
                                      sh->F, view_of(h), stream), "gate GEMM");
}

twell_status twell_sparse_up(const twell_ffn_shape* sh, const void* x, const void* WuT, const twell_mat* h,
                             float* aval, hipStream_t stream) {
  twell_status st = check_shape(sh);
  if (!st) st = check_tensors(sh, {x, WuT, aval});
  if (!st) st = check_h(sh, h);
  if (st) return st;
  if (sh->T == 0) return TWELL_OK;
  return hip_status(launch_sddmm_up(sh->in_dt == TWELL_BF16 ? DT_BF16 : DT_F32, x, WuT, sh->T, sh->d, sh->F,
                                    view_of(h), aval, nullptr, stream), "sparse up-projection");
}

twell_status twell_sparse_down(const twell_ffn_shape* sh, const float* aval, const void* Wd,
                               const twell_mat* pattern, void* y, hipStream_t stream) {
  twell_status st = check_shape(sh);
  if (!st) st = check_tensors(sh, {aval, Wd, y});
  if (!st) st = check_h(sh, pattern);
  if (st) return st;
  if (sh->T == 0) return TWELL_OK;
  return hip_status(launch_spmm_down(sh->in_dt == TWELL_BF16 ? DT_BF16 : DT_F32,
                                     sh->out_dt == TWELL_BF16 ? DT_BF16 : DT_F32, aval, Wd, sh->T, sh->d, sh->F,
                                     view_of(pattern), y, nullptr, stream), "sparse down-projection");
}

// ------------------------------------------------------------------ non-gated ReLU FFN

// Workspace of the non-gated forward: the TwELL of h (when the caller keeps
// none) and, for bf16 inputs, the union workspace.
static size_t relu_layout(const twell_ffn_shape* sh, void* ws, FwdWs* out) {
  size_t parts[5];
  mat_parts(sh->T, sh->F, GPU_R, GPU_C, TWELL_F32, parts);
  Carver c(ws);
  FwdWs w{};
  TwellView& v = w.h;
  v.T = sh->T; v.F = sh->F; v.NT = sh->F / GPU_C; v.NR = (sh->T + GPU_R - 1) / GPU_R;
  v.cnt = (uint8_t*)c.take(parts[0]);
  v.width = (uint8_t*)c.take(parts[1]);
  v.val = c.take(parts[2]);
  v.idx = (uint8_t*)c.take(parts[3]);
  v.mask = (uint64_t*)c.take(parts[4]);
  if (sh->in_dt == TWELL_BF16) w.uni = c.take(union_ws_bytes(sh->T, sh->d, sh->F));
  if (out) *out = w;
  return c.off;
}

size_t twell_relu_ffn_fwd_workspace(const twell_ffn_shape* sh) {
  if (!sh || check_shape(sh) != TWELL_OK) return 0;
  return relu_layout(sh, nullptr, nullptr);
}

twell_status twell_relu_ffn_fwd(const twell_ffn_shape* sh, const void* x, const void* W1T, const void* b1,
                                const void* W2, void* y, twell_mat* saved_h, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  twell_status st = check_shape(sh);
  if (st) return st;
  if (sh->T > 0 && (!x || !W1T || !W2 || !y)) return fail(TWELL_EINVAL, "NULL tensor argument");
  if (!aligned16(x) || !aligned16(W1T) || !aligned16(W2) || !aligned16(y) || !aligned16(b1))
    return fail(TWELL_EINVAL, "tensors must be 16-byte aligned");
  if (saved_h) {
    st = check_mat(saved_h, true);
    if (st) return st;
    if (saved_h->T != sh->T || saved_h->F != sh->F || saved_h->vdtype != TWELL_F32)
      return fail(TWELL_EINVAL, "saved_h must be T x F with fp32 values");
  }
  const size_t need = relu_layout(sh, nullptr, nullptr);
  if (!ws || ws_bytes < need) return fail(TWELL_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (sh->T == 0) return TWELL_OK;
  FwdWs w;
  relu_layout(sh, ws, &w);
  const int in_dt = sh->in_dt == TWELL_BF16 ? DT_BF16 : DT_F32;
  const int out_dt = sh->out_dt == TWELL_BF16 ? DT_BF16 : DT_F32;
  const TwellView h = saved_h ? view_of(saved_h) : w.h;
  uint64_t* slabs = nullptr;
  int* uflag = nullptr;
  if (in_dt == DT_BF16) union_slabs_and_flag(sh->T, sh->F, w.uni, &slabs, &uflag);
  hipError_t e = launch_gate_twell(in_dt, x, W1T, b1, sh->T, sh->d, sh->F, h, stream, slabs, uflag);
  if (e != hipSuccess) return hip_status(e, "gate GEMM");
  if (in_dt == DT_BF16) {
    // h (or W2) beyond the fp16 range: the down kernel takes the per-pair fp32 path
    e = launch_union_fwd(x, nullptr, W2, sh->T, sh->d, sh->F, h, nullptr, w.uni, y, out_dt, nullptr, stream, nullptr,
                         nullptr, true);
    if (e != hipSuccess) return hip_status(e, "union down GEMM");
  } else {
    e = launch_spmm_down(in_dt, out_dt, (const float*)h.val, W2, sh->T, sh->d, sh->F, h, y, nullptr, stream);
    if (e != hipSuccess) return hip_status(e, "sparse down-projection");
  }
  return TWELL_OK;
}

// The non-gated layer with the same capacities as twell_ffn_fwd_bounded.
static size_t relu_bounded_layout(const twell_ffn_shape* sh, int32_t W, int32_t ucap, void* ws, FwdWs* out) {
  size_t parts[6];
  cmat_parts(sh->T, sh->F, W, parts);
  Carver c(ws);
  FwdWs w{};
  TwellView& v = w.h;
  v.T = sh->T; v.F = sh->F; v.NT = sh->F / GPU_C; v.NR = (sh->T + GPU_R - 1) / GPU_R;
  v.cap = W;
  v.cnt = (uint8_t*)c.take(parts[0]);
  v.width = (uint8_t*)c.take(parts[1]);
  v.val = c.take(parts[2]);
  v.idx = (uint8_t*)c.take(parts[3]);
  v.mask = (uint64_t*)c.take(parts[4]);
  w.uni = c.take(union_ws_bytes(sh->T, sh->d, sh->F, ucap));
  if (out) *out = w;
  return c.off;
}

size_t twell_relu_ffn_fwd_bounded_workspace(const twell_ffn_shape* sh, int32_t tile_cap, int32_t union_cap) {
  if (!sh || check_shape(sh) != TWELL_OK || sh->in_dt != TWELL_BF16 || !bounded_caps_ok(sh, tile_cap, union_cap))
    return 0;
  return relu_bounded_layout(sh, tile_cap, union_cap, nullptr, nullptr);
}

twell_status twell_relu_ffn_fwd_bounded(const twell_ffn_shape* sh, const void* x, const void* W1T, const void* b1,
                                        const void* W2, void* y, int32_t tile_cap, int32_t union_cap,
                                        int32_t* n_over_blocks, void* ws, size_t ws_bytes, hipStream_t stream) {
  twell_status st = check_shape(sh);
  if (st) return st;
  if (sh->in_dt != TWELL_BF16) return fail(TWELL_EUNSUPPORTED, "the bounded forward takes bf16 inputs");
  if (!bounded_caps_ok(sh, tile_cap, union_cap))
    return fail(TWELL_EINVAL, "tile_cap=%d must be a multiple of 4 in 4..64 and union_cap=%d a multiple of 64 in "
                "64..F=%d", tile_cap, union_cap, sh->F);
  if (sh->T > 0 && (!x || !W1T || !W2 || !y)) return fail(TWELL_EINVAL, "NULL tensor argument");
  if (!aligned16(x) || !aligned16(W1T) || !aligned16(W2) || !aligned16(y) || !aligned16(b1))
    return fail(TWELL_EINVAL, "tensors must be 16-byte aligned");
  const size_t need = relu_bounded_layout(sh, tile_cap, union_cap, nullptr, nullptr);
  if (!ws || ws_bytes < need) return fail(TWELL_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  hipError_t e = hipSuccess;
  FwdWs w;
  relu_bounded_layout(sh, tile_cap, union_cap, ws, &w);
  if (sh->T > 0) {
    const int out_dt = sh->out_dt == TWELL_BF16 ? DT_BF16 : DT_F32;
    uint64_t* slabs = nullptr;
    int* uflag = nullptr;
    union_slabs_and_flag(sh->T, sh->F, w.uni, &slabs, &uflag);
    e = launch_gate_twell(DT_BF16, x, W1T, b1, sh->T, sh->d, sh->F, w.h, stream, slabs, uflag);
    if (e != hipSuccess) return hip_status(e, "gate GEMM");
    e = launch_union_fwd(x, nullptr, W2, sh->T, sh->d, sh->F, w.h, nullptr, w.uni, y, out_dt, nullptr, stream, nullptr,
                         nullptr, true, W1T, b1, union_cap);
    if (e != hipSuccess) return hip_status(e, "union down GEMM");
  }
  if (n_over_blocks) e = launch_union_over_count(sh->T, sh->F, w.uni, sh->T > 0 ? union_cap : 0, n_over_blocks, stream);
  return hip_status(e, "block count");
}

size_t twell_relu_ffn_dense_fwd_workspace(const twell_ffn_shape* sh) {
  if (!sh || check_shape(sh) != TWELL_OK) return 0;
  return round_up((size_t)sh->T * sh->F * 2, 256);
}

twell_status twell_relu_ffn_dense_fwd(const twell_ffn_shape* sh, const void* x, const void* W1T, const void* b1,
                                      const void* W2, void* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  twell_status st = check_shape(sh);
  if (st) return st;
  if (sh->in_dt != TWELL_BF16) return fail(TWELL_EUNSUPPORTED, "the dense baseline is bf16 only");
  if (sh->T > 0 && (!x || !W1T || !W2 || !y)) return fail(TWELL_EINVAL, "NULL tensor argument");
  if (!aligned16(x) || !aligned16(W1T) || !aligned16(W2) || !aligned16(y) || !aligned16(b1))
    return fail(TWELL_EINVAL, "tensors must be 16-byte aligned");
  if (sh->F % 128 != 0) return fail(TWELL_EUNSUPPORTED, "the dense baseline needs F %% 128 == 0");
  const size_t need = twell_relu_ffn_dense_fwd_workspace(sh);
  if (!ws || ws_bytes < need) return fail(TWELL_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (sh->T == 0) return TWELL_OK;
  return hip_status(launch_dense_relu_fwd(x, W1T, b1, W2, sh->T, sh->d, sh->F, ws,
                                          sh->out_dt == TWELL_BF16 ? DT_BF16 : DT_F32, y, stream),
                    "dense ReLU FFN");
}

// The dense baseline takes the few-token kernels where the TwELL forward does.
bool dense_few_tokens(const twell_ffn_shape* sh) { return sh->T > 0 && sh->T <= DECODE_T_MAX; }

size_t twell_ffn_dense_fwd_workspace(const twell_ffn_shape* sh) {
  if (!sh || check_shape(sh) != TWELL_OK) return 0;
  if (dense_few_tokens(sh)) return dense_few_ws_bytes(sh->T, sh->d, sh->F);
  return round_up((size_t)sh->T * sh->F * 2, 256);
}

twell_status twell_ffn_dense_fwd(const twell_ffn_shape* sh, const void* x, const void* WgT, const void* bg,
                                 const void* WuT, const void* Wd, void* y, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  twell_status st = check_shape(sh);
  if (st) return st;
  if (sh->in_dt != TWELL_BF16) return fail(TWELL_EUNSUPPORTED, "the dense baseline is bf16 only");
  if (sh->T > 0 && (!x || !WgT || !WuT || !Wd || !y)) return fail(TWELL_EINVAL, "NULL tensor argument");
  if (!aligned16(x) || !aligned16(WgT) || !aligned16(WuT) || !aligned16(Wd) || !aligned16(y) || !aligned16(bg))
    return fail(TWELL_EINVAL, "tensors must be 16-byte aligned");
  if (sh->F % 128 != 0) return fail(TWELL_EUNSUPPORTED, "the dense baseline needs F %% 128 == 0");
  const size_t need = twell_ffn_dense_fwd_workspace(sh);
  if (!ws || ws_bytes < need) return fail(TWELL_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (sh->T == 0) return TWELL_OK;
  if (dense_few_tokens(sh))
    return hip_status(launch_dense_few_fwd(x, WgT, bg, WuT, Wd, sh->T, sh->d, sh->F, ws,
                                           sh->out_dt == TWELL_BF16 ? DT_BF16 : DT_F32, y, stream),
                      "dense few-token FFN");
  return hip_status(launch_dense_fwd(x, WgT, bg, WuT, Wd, sh->T, sh->d, sh->F, ws,
                                     sh->out_dt == TWELL_BF16 ? DT_BF16 : DT_F32, y, stream),
                    "dense FFN");
}

size_t twell_ffn_dense_bwd_workspace(const twell_ffn_shape* sh) {
  if (!sh || check_shape(sh) != TWELL_OK) return 0;
  return dense_train_ws_bytes(sh->T, sh->d, sh->F);
}

twell_status twell_ffn_dense_bwd(const twell_ffn_shape* sh, const void* x, const void* WgT, const void* bg,
                                 const void* WuT, const void* Wd, const void* dY, void* y, float* dX, float* dWgT,
                                 float* dWuT, float* dWd, float* dbg, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  twell_status st = check_shape(sh);
  if (st) return st;
  if (sh->in_dt != TWELL_BF16) return fail(TWELL_EUNSUPPORTED, "the dense training baseline is bf16 only");
  if (!WgT || !WuT || !Wd || !dWgT || !dWuT || !dWd) return fail(TWELL_EINVAL, "NULL weight or gradient argument");
  if (sh->T > 0 && (!x || !dY || !y || !dX)) return fail(TWELL_EINVAL, "NULL tensor argument");
  for (const void* p : {x, WgT, bg, WuT, Wd, dY, (const void*)y, (const void*)dX, (const void*)dWgT,
                        (const void*)dWuT, (const void*)dWd, (const void*)dbg})
    if (!aligned16(p)) return fail(TWELL_EINVAL, "tensors must be 16-byte aligned");
  if (sh->T % 64 != 0 || sh->d % 256 != 0 || sh->F % 256 != 0)
    return fail(TWELL_EUNSUPPORTED, "the dense training baseline needs T %% 64 == 0, d %% 256 == 0, F %% 256 == 0");
  const size_t need = dense_train_ws_bytes(sh->T, sh->d, sh->F);
  if (!ws || ws_bytes < need) return fail(TWELL_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (sh->T == 0) {
    // no tokens: the weight gradients are zero
    const int64_t n = (int64_t)sh->F * sh->d;
    hipError_t e = launch_zero_f32(dWgT, n, stream);
    if (e == hipSuccess) e = launch_zero_f32(dWuT, n, stream);
    if (e == hipSuccess) e = launch_zero_f32(dWd, n, stream);
    if (e == hipSuccess) e = launch_zero_f32(dbg, sh->F, stream);
    return hip_status(e, "dense training baseline");
  }
  return hip_status(launch_dense_train(x, WgT, bg, WuT, Wd, dY, sh->T, sh->d, sh->F, ws,
                                       sh->out_dt == TWELL_BF16 ? DT_BF16 : DT_F32, y, dX, dWgT, dWuT, dWd, dbg,
                                       stream),
                    "dense training baseline");
}

// ------------------------------------------------------------------ forward without allocation

}  // extern "C"

namespace {

// Scratch of twell_ffn_fwd_noalloc: one static array per device, held until
// the process ends.  Host code never passes `scratch` itself to a kernel (on
// the host that name is a stand-in, not a device address); it uses the
// device address hipGetSymbolAddress returns, looked up once per device with
// that device current.
static_assert(TWELL_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
__device__ __align__(256) static char scratch[TWELL_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch[MAX_DEVICES] = {};

twell_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return fail(TWELL_EUNSUPPORTED, "device %d beyond the %d supported", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(TWELL_EHIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return TWELL_OK;
}

}  // namespace

extern "C" {

twell_status twell_ffn_fwd_noalloc(const twell_ffn_shape* sh, const void* x, const void* WgT, const void* bg,
                                   const void* WuT, const void* Wd, void* y, twell_mat* saved_h,
                                   int32_t dense_row_threshold, hipStream_t stream) {
  twell_status st = check_shape(sh);
  if (st) return st;
  const size_t need = fwd_layout(sh, dense_row_threshold >= 0, nullptr, nullptr);
  if (need > TWELL_NOALLOC_SCRATCH_BYTES)
    return fail(TWELL_EWORKSPACE, "this shape needs %zu bytes of scratch; the static scratch holds %zu",
                need, (size_t)TWELL_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st) return st;
  return twell_ffn_fwd_ex(sh, x, WgT, bg, WuT, Wd, y, saved_h, dense_row_threshold, ws,
                          TWELL_NOALLOC_SCRATCH_BYTES, stream, nullptr, 0);
}

const char* twell_status_string(twell_status st) {
  switch (st) {
    case TWELL_OK: return "ok";
    case TWELL_EINVAL: return "invalid argument";
    case TWELL_EUNSUPPORTED: return "unsupported by the GPU path";
    case TWELL_EWORKSPACE: return "workspace too small";
    case TWELL_EHIP: return "HIP error";
  }
  return "unknown status";
}

const char* twell_last_error(void) { return g_err; }

}  // extern "C"
