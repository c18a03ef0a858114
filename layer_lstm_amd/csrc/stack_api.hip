// stack_api.hip -- stacked layers (lstm_stack_* in include/lstm.h): the
// plan, the workspace layout and the wavefront schedule of the forward pass
// and the backpropagation through time of L one-direction layers, where
// layer l + 1 takes layer l's output sequence as its input (the MXNet
// page's "Stack Multiple RNN Cells"; the CMU 10-414 page's LSTM with
// num_layers).
//
// Wavefront.  Time is cut into C chunks.  In wave w of the forward, layer l
// runs chunk w - l: its input projection over the chunk (layer l - 1's
// output for that chunk is complete since wave w - 1; layer 0's projection
// runs once over all T before the first wave), then its recurrence over the
// chunk's steps, starting from the state the previous chunk left (h from the
// layer's output, c from its fp32 record).  The recurrences of a wave run in
// one persistent launch, each layer on its share of the compute units (a
// layout for cus / n when n layers are active), so layer l + 1's steps of
// chunk k run beside layer l's steps of chunk k + 1; a wave with one active
// layer gives it the whole device, and one chunk is plain layer-by-layer.
// The backward runs the waves from the last chunk of the last layer: layer
// l's chunk k needs its output cotangent for the chunk (the user's dy for
// the last layer, else the input gradient of layer l + 1 for the chunk,
// formed by the dx product right after that layer's recurrence over it) and
// the carries of its own chunk k + 1 (kept in fp32).  Layer 0's input
// gradient, and dW and db of every layer, are formed once at the end over
// all T*B rows.  The exchange regions of all layers lie side by side, so the
// one product launch a wave makes anyway clears them for the next wave.
#include <hip/hip_runtime.h>
#include <string.h>

#include "internal.hpp"
#include "lstm.h"

namespace lstm {

constexpr int kMaxLayers = 8;
constexpr int kStackSlots = 4;  // recurrences per launch (kMaxSlots)
constexpr int64_t kMinChunkSteps = 128, kMaxChunks = 8;

static size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

struct StackPlan {
  int L, C, Tc;
  int maxdiv;                     // most layers one launch runs (1: one after the other)
  Plan pl[2][kStackSlots + 1];    // [kind][d]: recurrences on cus / d; kind 0: layer 0 (input I), 1: input H
  bool ok[kStackSlots + 1];       // a layout on cus / d exists
  size_t hx_bytes, px_bytes;      // one layer's exchange regions (the largest of the layouts)
  int dbp_rows;                   // db partial rows of one chunk (the largest batch-group count)
  // workspace: error word, the layers' HX regions, their PX regions, their
  // db partials ([C][dbp_rows][4H] each), split-K partials of the products,
  // then one block per layer: P (fp32 projections, later the gate deltas),
  // G, C (fp32 cell record), y, dy, fp32 carries
  size_t off_hx, off_px, off_dbp, off_gp, off_blocks, block;
  size_t b_P, b_G, b_C, b_y, b_dy, b_carry;
  size_t total;
};

static Plan chunk_of(const Plan& full, int64_t tc) {
  Plan c = full;
  c.T = tc;
  c.TB = tc * full.B;
  return c;
}

static int stack_plan(const lstm_shape* shape, int64_t layers, int64_t chunks, StackPlan* sp) {
  if (!shape) return LSTM_ERR_NULL;
  if ((shape->flags & ~(LSTM_GATES_IJFO | LSTM_TWO_BIAS)) != 0) return LSTM_ERR_DTYPE;
  if (layers < 1 || layers > kMaxLayers || chunks < 0) return LSTM_ERR_DIMS;
  if (shape->T < 0 || shape->B < 0 || shape->I < 0 || shape->H <= 0) return LSTM_ERR_DIMS;
  memset(sp, 0, sizeof(*sp));
  const int L = (int)layers;
  const int64_t T = shape->T;
  // default: chunks of at least kMinChunkSteps steps, at most kMaxChunks
  // (shorter chunks pay more in the products' fixed costs than the overlap
  // of the layers' recurrences gains)
  int64_t C64 = chunks > 0 ? (chunks < T ? chunks : T) : T / kMinChunkSteps;
  if (chunks == 0 && C64 > kMaxChunks) C64 = kMaxChunks;
  int C = C64 < 1 ? 1 : (int)C64;
  const int64_t Tc = T > 0 ? (T + C - 1) / C : 1;
  C = T > 0 ? (int)((T + Tc - 1) / Tc) : 1;
  // the whole-device layouts, then one for cus / d for every d up to the
  // layers a wave can hold
  int rc = make_plan(T, shape->B, shape->I, shape->H, shape->dtype, &sp->pl[0][1], 1);
  if (rc == LSTM_OK) rc = make_plan(T, shape->B, shape->H, shape->H, shape->dtype, &sp->pl[1][1], 1);
  if (rc != LSTM_OK) return rc;
  sp->ok[1] = true;
  sp->maxdiv = 1;
  const int dmax = (L < C ? L : C) < kStackSlots ? (L < C ? L : C) : kStackSlots;
  for (int d = 2; d <= dmax; ++d) {
    int r = make_plan(T, shape->B, shape->I, shape->H, shape->dtype, &sp->pl[0][d], d);
    if (r == LSTM_OK) r = make_plan(T, shape->B, shape->H, shape->H, shape->dtype, &sp->pl[1][d], d);
    if (r == LSTM_OK) {
      sp->ok[d] = true;
      sp->maxdiv = d;
    } else if (r != LSTM_ERR_UNSUPPORTED) {
      return r;
    }
  }
  const int flags_ijfo = (shape->flags & LSTM_GATES_IJFO) ? 1 : 0, flags_tb = (shape->flags & LSTM_TWO_BIAS) ? 1 : 0;
  for (int d = 1; d <= kStackSlots; ++d) {
    if (!sp->ok[d]) continue;
    for (int i = 0; i < 2; ++i) {
      Plan& q = sp->pl[i][d];
      q.ijfo = flags_ijfo;
      q.two_bias = flags_tb;
      if (q.bytes_HX > sp->hx_bytes) sp->hx_bytes = q.bytes_HX;
      if (q.bytes_PX > sp->px_bytes) sp->px_bytes = q.bytes_PX;
      if (q.nBG > sp->dbp_rows) sp->dbp_rows = q.nBG;
    }
  }
  sp->L = L;
  sp->C = C;
  sp->Tc = (int)Tc;
  // split-K partials: the whole-T products of both layer kinds, the chunk
  // products of layers >= 1 (all on the whole device)
  size_t gp = 0;
  for (int i = 0; i < 2; ++i) {
    const Plan& f = sp->pl[i][1];
    const size_t g0 = gemm_partial_bytes(f, f.cus);
    const size_t g1 = gemm_partial_bytes(chunk_of(f, Tc), f.cus);
    const size_t g2 = T > 0 ? gemm_partial_bytes(chunk_of(f, T - (int64_t)(C - 1) * Tc), f.cus) : 0;
    if (g0 > gp) gp = g0;
    if (g1 > gp) gp = g1;
    if (g2 > gp) gp = g2;
  }
  const Plan& a = sp->pl[0][1];
  const int e = a.esize;
  sp->off_hx = 256;
  sp->off_px = sp->off_hx + (size_t)L * sp->hx_bytes;
  sp->off_dbp = sp->off_px + (size_t)L * sp->px_bytes;
  sp->off_gp = sp->off_dbp + al256((size_t)L * C * sp->dbp_rows * a.G4 * 4);
  sp->off_blocks = sp->off_gp + al256(gp);
  sp->b_P = 0;
  sp->b_G = sp->b_P + al256((size_t)a.TB * a.G4 * 4);
  sp->b_C = sp->b_G + al256((size_t)a.TB * a.G4 * e);
  sp->b_y = sp->b_C + al256((size_t)a.TB * a.H * 4);
  sp->b_dy = sp->b_y + al256((size_t)a.TB * a.H * e);
  sp->b_carry = sp->b_dy + al256((size_t)a.TB * a.H * e);
  sp->block = sp->b_carry + al256((size_t)2 * a.B * a.H * 4);
  sp->total = sp->off_blocks + (size_t)L * sp->block;
  return LSTM_OK;
}

// Launch groups of a wave's n recurrences: `size` slots a launch on the
// layout for cus / div.
static void wave_groups(const StackPlan& sp, int n, int* size, int* div) {
  int g = n < sp.maxdiv ? n : sp.maxdiv;
  while (g > 1 && !sp.ok[g]) --g;
  *size = g;
  *div = g;
}

static bool misal(const void* ptr, int esize) { return ptr && ((uintptr_t)ptr % (uintptr_t)esize) != 0; }

static int status_from(hipError_t e) {
  if (e == hipSuccess) return LSTM_OK;
  if (e == hipErrorCooperativeLaunchTooLarge) return LSTM_ERR_COOP;
  return LSTM_ERR_LAUNCH;
}

}  // namespace lstm

using namespace lstm;

extern "C" {

int lstm_stack_query(const lstm_shape* shape, int64_t layers, int64_t chunks, size_t* workspace_bytes,
                     int32_t* concurrent) {
  if (!shape || !workspace_bytes) return LSTM_ERR_NULL;
  StackPlan sp;
  const int rc = stack_plan(shape, layers, chunks, &sp);
  if (rc != LSTM_OK) return rc;
  *workspace_bytes = sp.total;
  if (concurrent) *concurrent = sp.maxdiv;
  return LSTM_OK;
}

int lstm_stack_fwd_train(const lstm_shape* shape, int64_t layers, int64_t chunks, const void* x, const void* W,
                         const void* b, const void* h0, const void* c0, void* y, void* hT, void* cT, void* workspace,
                         size_t workspace_bytes, void* stream) {
  StackPlan sp;
  const int rc = stack_plan(shape, layers, chunks, &sp);
  if (rc != LSTM_OK) return rc;
  const Plan& p0 = sp.pl[0][1];
  const int e = p0.esize, L = sp.L;
  const int64_t T = p0.T, B = p0.B, H = p0.H, I = p0.I, G4 = p0.G4;
  if (!W || !workspace) return LSTM_ERR_NULL;
  if (T * B * I > 0 && !x) return LSTM_ERR_NULL;
  if (T * B > 0 && !y) return LSTM_ERR_NULL;
  if (B > 0 && (!hT || !cT)) return LSTM_ERR_NULL;
  if (misal(x, e) || misal(W, e) || misal(b, e) || misal(h0, e) || misal(c0, e) || misal(y, e) || misal(hT, e) ||
      misal(cT, e) || ((uintptr_t)workspace & 255u))
    return LSTM_ERR_ALIGN;
  if (workspace_bytes < sp.total) return LSTM_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  hipError_t err = hipSuccess;
  const int64_t sst = B * H * e;
  if (B == 0 || T == 0) {
    // no recurrence runs: the status word is cleared here (see lstm_fwd_train)
    err = launch_fill_zero(ws, 4, s);
    if (err == hipSuccess && B > 0) err = launch_copy_state(h0, hT, (size_t)(L * B * H), e, s);
    if (err == hipSuccess && B > 0) err = launch_copy_state(c0, cT, (size_t)(L * B * H), e, s);
    return status_from(err);
  }
  auto wof = [&](int l) -> const char* {
    return (const char*)W + (l == 0 ? 0 : (G4 * (H + I) + (int64_t)(l - 1) * G4 * 2 * H) * e);
  };
  const int64_t bst = (p0.two_bias ? 2 : 1) * G4 * e;
  auto blk = [&](int l) { return ws + sp.off_blocks + (size_t)l * sp.block; };
  auto yof = [&](int l) -> char* { return l == L - 1 ? (char*)y : blk(l) + sp.b_y; };
  auto at = [](const void* q, int64_t off) -> const char* { return q ? (const char*)q + off : nullptr; };
  uint32_t* errw = (uint32_t*)ws;
  float* gp = (float*)(ws + sp.off_gp);
  const size_t hx_all = (size_t)L * sp.hx_bytes;

  // layer 0's projection over all T; the launch clears the error word and
  // every layer's exchange region
  {
    Timed tm(0, s);
    err = launch_gemm_inproj(p0, x, wof(0), b, (float*)(blk(0) + sp.b_P), gp, ws, sp.off_hx + hx_all, s);
  }
  const int waves = sp.C + L - 1;
  for (int w = 0; w < waves && err == hipSuccess; ++w) {
    FwdSlot sl[kMaxLayers];
    int ns = 0;
    bool cleared = w == 0;
    for (int l = 0; l < L && err == hipSuccess; ++l) {
      const int k = w - l;
      if (k < 0 || k >= sp.C) continue;
      const int64_t t0 = (int64_t)k * sp.Tc, tc = (T - t0) < sp.Tc ? (T - t0) : sp.Tc;
      const int64_t Il = l == 0 ? I : H;
      char* bl = blk(l);
      if (l > 0) {
        // the chunk's projection of the layer below's output; the first of
        // the wave clears the exchange regions
        Timed tm(0, s);
        err = launch_gemm_inproj(chunk_of(sp.pl[1][1], tc), yof(l - 1) + t0 * B * H * e, wof(l), at(b, l * bst),
                                 (float*)(bl + sp.b_P) + t0 * B * G4, gp, cleared ? nullptr : ws + sp.off_hx,
                                 cleared ? 0 : hx_all, s);
        cleared = true;
      }
      sl[ns++] = FwdSlot{(const float*)(bl + sp.b_P) + t0 * B * G4,
                         wof(l),
                         H + Il,
                         k == 0 ? at(h0, l * sst) : yof(l) + (t0 - 1) * B * H * e,
                         k == 0 ? at(c0, l * sst) : nullptr,
                         k == 0 ? nullptr : (const float*)(bl + sp.b_C) + (t0 - 1) * B * H,
                         yof(l) + t0 * B * H * e,
                         (char*)hT + l * sst,
                         (char*)cT + l * sst,
                         bl + sp.b_G + t0 * B * G4 * e,
                         (float*)(bl + sp.b_C) + t0 * B * H,
                         (uint64_t*)(ws + sp.off_hx + (size_t)l * sp.hx_bytes),
                         (int)tc,
                         0};
    }
    if (err == hipSuccess && !cleared) err = launch_fill_zero(ws + sp.off_hx, hx_all, s);
    // the wave's recurrences, as many a launch as a layout for them exists
    // (layers 0 and >= 1 share the layout)
    int g = 1, d = 1;
    wave_groups(sp, ns, &g, &d);
    for (int i = 0; i < ns && err == hipSuccess; i += g) {
      const int r = ns - i < g ? ns - i : g;
      Timed tm(1, s);
      err = launch_fwd_recurrent(sp.pl[1][sp.ok[r] ? r : d], sl + i, r, errw, nullptr, nullptr, s);
    }
  }
  return status_from(err);
}

int lstm_stack_bwd(const lstm_shape* shape, int64_t layers, int64_t chunks, const void* dy, const void* dhT,
                   const void* dcT, const void* x, const void* W, const void* h0, const void* c0, const void* y,
                   void* workspace, size_t workspace_bytes, void* dx, void* dW, void* db, void* dh0, void* dc0,
                   void* stream) {
  StackPlan sp;
  const int rc = stack_plan(shape, layers, chunks, &sp);
  if (rc != LSTM_OK) return rc;
  const Plan& p0 = sp.pl[0][1];
  const int e = p0.esize, L = sp.L;
  const int64_t T = p0.T, B = p0.B, H = p0.H, I = p0.I, G4 = p0.G4;
  if (!W || !dW || !workspace) return LSTM_ERR_NULL;
  if (T * B > 0 && (!dy || !y)) return LSTM_ERR_NULL;
  if (T * B * I > 0 && (!x || !dx)) return LSTM_ERR_NULL;
  if (B > 0 && (!dh0 || !dc0)) return LSTM_ERR_NULL;
  if (misal(dy, e) || misal(dhT, e) || misal(dcT, e) || misal(x, e) || misal(W, e) || misal(h0, e) ||
      misal(c0, e) || misal(y, e) || misal(dx, e) || misal(dW, e) || misal(db, e) || misal(dh0, e) ||
      misal(dc0, e) || ((uintptr_t)workspace & 255u))
    return LSTM_ERR_ALIGN;
  if (workspace_bytes < sp.total) return LSTM_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  hipError_t err = hipSuccess;
  const int64_t sst = B * H * e, bst = (p0.two_bias ? 2 : 1) * G4 * e;
  const int64_t wtot = (G4 * (H + I) + (int64_t)(L - 1) * G4 * 2 * H) * e;
  if (T == 0 || B == 0) {
    err = launch_fill_zero(dW, (size_t)wtot, s);
    if (err == hipSuccess && db) err = launch_fill_zero(db, (size_t)(L * bst), s);
    if (err == hipSuccess && B > 0) err = launch_copy_state(dhT, dh0, (size_t)(L * B * H), e, s);
    if (err == hipSuccess && B > 0) err = launch_copy_state(dcT, dc0, (size_t)(L * B * H), e, s);
    return status_from(err);
  }
  auto woff = [&](int l) -> int64_t { return l == 0 ? 0 : (G4 * (H + I) + (int64_t)(l - 1) * G4 * 2 * H) * e; };
  auto blk = [&](int l) { return ws + sp.off_blocks + (size_t)l * sp.block; };
  auto yof = [&](int l) -> const char* { return l == L - 1 ? (const char*)y : blk(l) + sp.b_y; };
  auto xof = [&](int l) -> const char* { return l == 0 ? (const char*)x : yof(l - 1); };
  // output cotangent of layer l: the user's for the last layer, else the
  // input gradient of the layer above
  auto dyof = [&](int l) -> char* { return l == L - 1 ? (char*)dy : blk(l) + sp.b_dy; };
  auto dbp = [&](int l) { return (float*)(ws + sp.off_dbp) + (int64_t)l * sp.C * sp.dbp_rows * G4; };
  auto at = [](const void* q, int64_t off) -> const char* { return q ? (const char*)q + off : nullptr; };
  uint32_t* errw = (uint32_t*)ws;
  float* gp = (float*)(ws + sp.off_gp);
  const size_t px_all = (size_t)L * sp.px_bytes;

  // error word, exchange regions and db partials (rows a chunk's layout does
  // not fill stay zero)
  err = launch_fill_zero(ws, sp.off_gp, s);
  const int waves = sp.C + L - 1;
  for (int w = 0; w < waves && err == hipSuccess; ++w) {
    BwdSlot sl[kMaxLayers];
    int lay[kMaxLayers], chk[kMaxLayers];
    int ns = 0;
    for (int l = L - 1; l >= 0; --l) {
      const int k = (sp.C - 1) - (w - (L - 1 - l));
      if (k < 0 || k >= sp.C) continue;
      const int64_t t0 = (int64_t)k * sp.Tc, tc = (T - t0) < sp.Tc ? (T - t0) : sp.Tc;
      char* bl = blk(l);
      lay[ns] = l;
      chk[ns] = k;
      sl[ns++] = BwdSlot{(const char*)W + woff(l),
                         H + (l == 0 ? I : H),
                         k == 0 ? at(c0, l * sst) : nullptr,
                         k == 0 ? nullptr : (const float*)(bl + sp.b_C) + (t0 - 1) * B * H,
                         dyof(l) + t0 * B * H * e,
                         k == sp.C - 1 ? at(dhT, l * sst) : nullptr,
                         k == sp.C - 1 ? at(dcT, l * sst) : nullptr,
                         bl + sp.b_G + t0 * B * G4 * e,
                         (const float*)(bl + sp.b_C) + t0 * B * H,
                         bl + sp.b_P + t0 * B * G4 * e,
                         (uint64_t*)(ws + sp.off_px + (size_t)l * sp.px_bytes),
                         db ? dbp(l) + (int64_t)k * sp.dbp_rows * G4 : nullptr,
                         (char*)dh0 + l * sst,
                         (char*)dc0 + l * sst,
                         (float*)(bl + sp.b_carry),
                         k < sp.C - 1 ? 1 : 0,
                         k > 0 ? 1 : 0,
                         (int)tc,
                         0};
    }
    int g = 1, d = 1;
    wave_groups(sp, ns, &g, &d);
    for (int i = 0; i < ns && err == hipSuccess; i += g) {
      const int r = ns - i < g ? ns - i : g;
      Timed tm(2, s);
      err = launch_bwd_recurrent(sp.pl[1][sp.ok[r] ? r : d], sl + i, r, errw, nullptr, nullptr, s);
    }
    // the input gradients of layers >= 1 over their chunks (the output
    // cotangents of the layers below for the next wave); the first clears
    // the exchange regions for the next wave
    const bool last = w == waves - 1;
    bool cleared = last;
    for (int i = 0; i < ns && err == hipSuccess; ++i) {
      const int l = lay[i], k = chk[i];
      if (l == 0) continue;
      const int64_t t0 = (int64_t)k * sp.Tc, tc = (T - t0) < sp.Tc ? (T - t0) : sp.Tc;
      Timed tm(4, s);
      err = launch_gemm_dx(chunk_of(sp.pl[1][1], tc), blk(l) + sp.b_P + t0 * B * G4 * e, (const char*)W + woff(l),
                           dyof(l - 1) + t0 * B * H * e, gp, cleared ? nullptr : ws + sp.off_px, cleared ? 0 : px_all,
                           s);
      cleared = true;
    }
    if (err == hipSuccess && !cleared) err = launch_fill_zero(ws + sp.off_px, px_all, s);
  }
  // layer 0's input gradient over all T
  if (err == hipSuccess && I > 0) {
    Timed tm(4, s);
    err = launch_gemm_dx(p0, blk(0) + sp.b_P, W, dx, gp, nullptr, 0, s);
  }
  // dW and db of each layer over all T*B rows
  for (int l = 0; l < L && err == hipSuccess; ++l) {
    Plan pf = sp.pl[l == 0 ? 0 : 1][1];
    pf.dbp_rows = sp.C * sp.dbp_rows;
    Timed tm(3, s);
    err = launch_gemm_dw(pf, blk(l) + sp.b_P, xof(l), at(h0, l * sst), yof(l), (char*)dW + woff(l), gp, nullptr, 0,
                         dbp(l), db ? (char*)db + l * bst : nullptr, s);
  }
  return status_from(err);
}

}  // extern "C"
