// Internal host-side interface between the C-ABI entry points and the kernel
// translation units.  Not part of the public header.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace twell {

enum { DT_F32 = 0, DT_BF16 = 1 };

// Compute units of the current device (persistent grids are sized by it).
inline int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    return 256;
  return n;
}

// Device view of a TwELL matrix (all pointers device memory).
struct TwellView {
  int T, F, NT, NR;
  uint8_t* cnt;     // [T][NT]
  uint8_t* width;   // [NR][NT]
  void* val;        // [NR][NT][cap][16]
  uint8_t* idx;     // [NR][NT][cap][16]
  uint64_t* mask;   // [T][NT] or null
  int cap = 64;     // slots per tile in val and idx; a tile wider than cap keeps
                    // its first cap slots (width still records the true width)
};

// Gate GEMM g = x.WgT^T + bg, h = ReLU(g), packed into TwELL in the epilogue
// (values fp32).  row_skip (optional, u8 [T]) marks rows whose mask must be
// stored as empty for the consumers (never used by the gate itself).
// slabs (bf16 only; nullable): the epilogue also writes the union of every
// 64-row slab's masks, slabs[t / 64][j], and workgroup 0 clears *flag.
hipError_t launch_gate_twell(int in_dt, const void* x, const void* WgT, const void* bg,
                             int T, int d, int F, const TwellView& out, hipStream_t s,
                             uint64_t* slabs = nullptr, int* flag = nullptr);

// Standalone pack of a [T][F] matrix with leading dimension ldg.
hipError_t launch_pack(const void* G, int gdt, int64_t ldg, const TwellView& out, hipStream_t s);
// Unpack to a dense [T][F] matrix with leading dimension ldh (value dtype vdt).
hipError_t launch_unpack(const TwellView& in, int vdt, void* H, int64_t ldh, hipStream_t s);

// Sparse up-projection times gate on the TwELL pattern:
//   a[t,n] = h[t,n] * (x_t . WuT[n]) for every stored (t, n), written into
//   aval (same layout as the TwELL values, fp32; may alias the h values).
// Rows with skip[t] != 0 are left untouched.
hipError_t launch_sddmm_up(int in_dt, const void* x, const void* WuT, int T, int d, int F,
                           const TwellView& h, float* aval, const uint8_t* skip, hipStream_t s);

// Sparse down-projection: y_t = sum over stored n of a[t,n] * Wd[n]
// (out_dt fp32 or bf16).  Rows with skip[t] != 0 are not written.
hipError_t launch_spmm_down(int in_dt, int out_dt, const float* aval, const void* Wd, int T,
                            int d, int F, const TwellView& pat, void* y, const uint8_t* skip,
                            hipStream_t s);

// Backward SDDMM on the pattern of h (rows with skip[t] != 0 untouched):
//   u = x_t.WuT[n], da = dY_t.Wd[n];  a = h*u, dg = da*u + l1, du = da*h
// written at the TwELL slot positions of h into aval, dgval, duval (l1: the
// activation penalty's gradient coefficient, added on every stored pair).
hipError_t launch_sddmm_bwd(int in_dt, const void* x, const void* dY, const void* WuT, const void* Wd, int T,
                            int d, int F, const TwellView& h, float* aval, float* dgval, float* duval,
                            const uint8_t* skip, hipStream_t s, float l1 = 0.f);

// The same for bf16 inputs as MFMA GEMMs over each 128-row block's union of
// the live rows' active neurons (rows with skip[t] != 0 excluded), followed by
// dX of the live rows = dG.WgT + dU.WuT as an fp16 MFMA GEMM over the same
// unions (dG, dU and the weights in fp16).  *flag_out receives the device flag
// that is set when a value exceeds the fp16 range: the dX GEMM then stands
// down and the per-pair dX kernel gated on the flag must run.  ws holds
// union_bwd_ws_bytes(T, d, F) bytes.
size_t union_bwd_ws_bytes(int T, int d, int F);
hipError_t launch_union_bwd(const void* x, const void* dY, const void* WgT, const void* WuT, const void* Wd, int T,
                            int d, int F, const TwellView& h, const uint8_t* skip, void* ws, float* aval,
                            float* dgval, float* duval, float l1, float* dX, int** flag_out, hipStream_t s);

// Backward SpMM: dX_t = sum over stored n of dg*WgT[n] + du*WuT[n] (fp32),
// rows with skip[t] != 0 not written.
hipError_t launch_spmm_dx(int in_dt, const float* dgval, const float* duval, const void* WgT, const void* WuT,
                          int T, int d, int F, const TwellView& pat, float* dX, const uint8_t* skip,
                          hipStream_t s);

// Compact TwELL (capacity W per (row, tile)) <-> the capacity-64 form; see
// twell_compact.hip.  Full side: cnt, width, val (fp32), idx, mask; compact
// side: ccnt, cwidth, cval, cidx, cmask, ovf (flags written when compacting).
struct CompactArgs {
  int T, NT, W;
  int64_t ntiles;
  uint8_t* cnt;
  uint8_t* width;
  float* val;
  uint8_t* idx;
  uint64_t* mask;
  uint8_t* ccnt;
  uint8_t* cwidth;
  float* cval;
  uint8_t* cidx;
  uint64_t* cmask;
  uint8_t* ovf;
};
hipError_t launch_compact(const CompactArgs& a, bool expand, hipStream_t s);
// The compact arrays (ccnt, cwidth, ovf, W, T, NT, ntiles) after a gate GEMM
// packed into them directly: ovf[t] = some ccnt[t][j] > W, widths clamped to W.
hipError_t launch_compact_finish(const CompactArgs& a, hipStream_t s);

// Row classification of the hybrid format: flag[t] = (sum_j cnt[t][j] > tau)
// or force[t] (force may be null);
// list[0..n) = flagged rows ascending; *n_out = n (and *n_copy if non-null).
hipError_t launch_classify(const TwellView& h, int tau, uint8_t* flag, int* list, int* n_out, int* n_copy,
                           hipStream_t s, const uint8_t* force = nullptr);

// Rows per round of the dense-row branch: its buffers hold this many rows and
// it runs in ceil(T / cap) rounds over the dense-row list (all of T up to
// 1024 tokens, else half of T rounded up to 128 rows: two rounds at most).
inline int dense_row_cap(int T) {
  if (T <= 1024) return T;
  const int h = (T + 1) / 2;
  return (h + 127) / 128 * 128;
}

// Dense-branch forward on the listed rows: actbuf [T][F] (rows < n used)
// receives ReLU(g)*u, then y[list[r]] = actbuf[r].Wd.
hipError_t launch_dense_rows_fwd(int in_dt, const void* x, const void* WgT, const void* bg, const void* WuT,
                                 const void* Wd, int T, int d, int F, const int* rows, const int* n_rows,
                                 float* actbuf, int out_dt, void* y, hipStream_t s);

// Dense-branch backward on the listed rows: buf3 [T][3F] receives [dG|dU|A];
// dX[list[r]] written; dWgT, dWuT, dWd (and dbg if non-null) are WRITTEN with
// the dense rows' contributions (zero when there are none).  dbg_part is
// [ceil(T/64)][F] scratch.
hipError_t launch_dense_rows_bwd(int in_dt, const void* x, const void* WgT, const void* bg, const void* WuT,
                                 const void* Wd, const void* dY, int T, int d, int F, const int* rows,
                                 const int* n_rows, float* buf3, float* dbg_part, float* dX, float* dWgT,
                                 float* dWuT, float* dWd, float* dbg, hipStream_t s, float l1 = 0.f);

// Sparse-branch weight gradients, ADDED to dWgT, dWuT, dWd (and dbg): a
// column-major index of the stored pairs of rows with skip[t] == 0 is built
// (part: [ceil(T/256)][F] ints, start: [F+1] ints, entries: one u32 per
// pair), then per neuron the sums over its tokens in ascending order.
hipError_t launch_sparse_wgrad(int in_dt, const void* x, const void* dY, int T, int d, int F,
                               const TwellView& h, const uint8_t* skip, int* part, int* start,
                               uint32_t* entries, const float* aval, const float* dgval, const float* duval,
                               float* dWgT, float* dWuT, float* dWd, float* dbg, hipStream_t s);

// bf16 sparse kernels with workgroup-shared weight staging (dY == null:
// forward up-projection; otherwise the backward's u/da products).
// gate: null, or a device flag; the kernels do nothing unless it is non-zero.
hipError_t launch_up_bf16(const void* x, const void* dY, const void* WuT, const void* Wd, int T, int d, int F,
                          const TwellView& h, float* aval, float* dgval, float* duval, const uint8_t* skip,
                          hipStream_t s, const int* gate = nullptr, float l1 = 0.f);
// y = v0 . W (+ v1 . W2 when v1 != null) over the stored pairs of pat.
hipError_t launch_down_bf16(const float* v0, const float* v1, const void* W, const void* W2, int T, int d, int F,
                            const TwellView& pat, void* y, int out_dt, const uint8_t* skip, hipStream_t s,
                            const int* gate = nullptr);

// Forward up/down over each 128-token row block's union of active neurons
// (bf16 inputs): union lists, up GEMM writing a as fp16 over the union, down
// GEMM into y (rows with skip[t] != 0 untouched).  ws holds
// union_ws_bytes(T, d, F).  *flag_out receives the device flag that is set when
// an a value overflows fp16; the caller then runs the pattern kernels gated on
// it (they recompute and overwrite y).
// ucap > 0: a holds ucap union positions per row (a multiple of 64, <= F);
// a block whose union is longer, or whose TwELL tiles are wider than h.cap,
// is computed per stored pair by the down kernel (h recomputed from WgT, bg).
size_t union_ws_bytes(int T, int d, int F, int ucap = 0);
// The leading part of that workspace the union lists alone use (lists,
// counts, flag, slab unions): all the few-token path needs.
size_t union_lists_ws_bytes(int T, int F);
// The union lists alone (for the few-token path), in the same workspace:
// pointers to the list and count of row block 0, and the two list kernels.
// slabs: the 64-row slab unions u64 [ceil(T/64)][F/64] the list kernel reads;
// with slabs_ready the caller has filled them and only the list kernel runs.
void union_lists_only(int T, int F, const TwellView& h, void* ws, int** ulist, int** ucount, uint64_t** slabs);
hipError_t launch_union_lists(int T, int F, const TwellView& h, void* ws, hipStream_t s, bool slabs_ready = false);

// Forward for few tokens (T <= DECODE_T_MAX, bf16, inference): the gate GEMM
// split along K over many workgroups with fixed-order partial sums, then one
// kernel for the TwELL pack of ReLU(g) into h and the up-projection of every
// stored pair, and one for the down-projection, both in fp32 (a kept in the
// TwELL layout inside ws).  ws holds decode_ws_bytes(T, d, F) bytes.  Events
// (nullable) after the gate GEMM, right after it again (the place of the
// union lists, which this path does not build), and after the pack and
// up-projection.
constexpr int DECODE_T_MAX = 256;
size_t decode_ws_bytes(int T, int d, int F);
hipError_t launch_decode_fwd(const void* x, const void* WgT, const void* bg, const void* WuT, const void* Wd, int T,
                             int d, int F, const TwellView& h, void* ws, void* y, int out_dt, hipStream_t s,
                             hipEvent_t ev_gate, hipEvent_t ev_lists, hipEvent_t ev_up);

// ev_lists / ev_up (nullable) are recorded after the union lists and the fp16
// copy of Wd, and after the up-projection.  WuT == null: the non-gated ReLU FFN
// (a = h, no up GEMM; x is not read).
hipError_t launch_union_fwd(const void* x, const void* WuT, const void* Wd, int T, int d, int F,
                            const TwellView& h, const uint8_t* skip, void* ws, void* y, int out_dt,
                            int** flag_out, hipStream_t s, hipEvent_t ev_lists = nullptr,
                            hipEvent_t ev_up = nullptr, bool slabs_ready = false, const void* WgT = nullptr,
                            const void* bg = nullptr, int ucap = 0);
// Writes to *out (device) the number of row blocks the last bounded forward
// in ws (union_ws_bytes(T, d, F, ucap > 0)) computed per pair; 0 for ucap <= 0.
hipError_t launch_union_over_count(int T, int F, void* ws, int ucap, int* out, hipStream_t s);
// The union workspace's slab unions and fp16-overflow flag, for a gate GEMM
// that writes the former and clears the latter (then launch_union_fwd runs
// with slabs_ready and skip == nullptr).
void union_slabs_and_flag(int T, int F, void* ws, uint64_t** slabs, int** flag);

// Dense non-gated ReLU FFN baseline: act = bf16(ReLU(x.W1T^T + b1)), then
// y = act.W2.  act is a [T][F] bf16 workspace; needs F % 128 == 0.
hipError_t launch_dense_relu_fwd(const void* x, const void* W1T, const void* b1, const void* W2, int T, int d, int F,
                                 void* act, int out_dt, void* y, hipStream_t s);

// Dense baseline: act = ReLU(x.WgT^T + bg) * (x.WuT^T) in bf16 (fused dual GEMM),
// then y = act.Wd.  act is a [T][F] bf16 workspace.
hipError_t launch_dense_fwd(const void* x, const void* WgT, const void* bg, const void* WuT,
                            const void* Wd, int T, int d, int F, void* act, int out_dt, void* y,
                            hipStream_t s);
// Dense baseline for few tokens (T <= DECODE_T_MAX), from the same split-K
// blocks as the few-token TwELL forward: gate and up partials in one GEMM,
// act = bf16(ReLU(g + b) * u), the split-K down-projection.
// ws: dense_few_ws_bytes(T, d, F).
size_t dense_few_ws_bytes(int T, int d, int F);
hipError_t launch_dense_few_fwd(const void* x, const void* WgT, const void* bg, const void* WuT, const void* Wd,
                                int T, int d, int F, void* ws, int out_dt, void* y, hipStream_t s);
// y = act.Wd for a bf16 act [T][F].
hipError_t launch_dense_down(const void* act, const void* Wd, int T, int d, int F, int out_dt, void* y,
                             hipStream_t s);

// Dense training step (forward + backward, bf16 intermediates): writes y and
// the fp32 gradients; dbg may be null.  Needs T % 64 == 0, d % 256 == 0,
// F % 256 == 0; workspace dense_train_ws_bytes(T, d, F).
size_t dense_train_ws_bytes(int T, int d, int F);
// p[0..n) = 0 with a kernel (no memset node, so the call can be graph-captured).
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s);
hipError_t launch_dense_train(const void* x, const void* WgT, const void* bg, const void* WuT, const void* Wd,
                              const void* dY, int T, int d, int F, void* ws, int out_dt, void* y, float* dX,
                              float* dWgT, float* dWuT, float* dWd, float* dbg, hipStream_t s);

}  // namespace twell
