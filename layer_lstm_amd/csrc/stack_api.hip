// stack_api.hip -- stacked layers (lstm_stack_* in include/lstm.h): the
// plan, the workspace layout and the wavefront schedule of the forward pass
// and the backpropagation through time of L one-direction layers, where
// layer l + 1 takes layer l's output sequence as its input (the MXNet
// page's "Stack Multiple RNN Cells"; the CMU 10-414 page's LSTM with
// num_layers).
//
// Wavefront.  Time is cut into C chunks.  In wave w of the forward, layer l
// runs chunk w - l: its input projection over the chunk (its input -- x, or
// the layer below's output -- for that chunk is complete since wave w - 1),
// then its recurrence over the chunk's steps, starting from the state the
// previous chunk left (h from the layer's output, c from its fp32 record).
// The recurrences of a wave run in one persistent launch, each layer on its
// share of the compute units (a layout for cus / L), so layer l + 1's steps
// of chunk k run beside layer l's steps of chunk k + 1.  The backward runs
// the waves from the last chunk of the last layer: layer l's chunk k needs
// its output cotangent for the chunk (the user's dy for the last layer, else
// the input gradient of layer l + 1 for the chunk, formed by the dx product
// right after that layer's recurrence over it) and the carries of its own
// chunk k + 1 (kept in fp32).  dW and db of each layer are formed once at
// the end over all T*B rows.  Where no layout for cus / L exists, the
// recurrences of a wave run one after the other on all compute units.
#include <hip/hip_runtime.h>
#include <string.h>

#include "internal.hpp"
#include "lstm.h"

namespace lstm {

constexpr int kMaxLayers = 8;
constexpr int kStackSlots = 4;  // recurrences per launch (kMaxSlots)

static size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

struct StackPlan {
  int L, C, Tc;
  int concurrent;           // the recurrences of a wave in one launch
  Plan pl[2];               // layer 0 (input size I) and layers >= 1 (input size H), whole T
  size_t off_block[kMaxLayers + 1];
  // inside a layer's block: the one-layer regions (ctrl, HX, PX, P / dG, G,
  // C at the plan's offsets), then these
  size_t off_gp, off_dbp, off_y, off_dy, off_carry;
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
  int C = chunks > 0 ? (int)(chunks < T ? chunks : (T > 0 ? T : 1)) : (int)(T < 8 ? (T > 0 ? T : 1) : 8);
  if (C < 1) C = 1;
  const int64_t Tc = T > 0 ? (T + C - 1) / C : 1;
  C = T > 0 ? (int)((T + Tc - 1) / Tc) : 1;
  // a layout of the recurrences on cus / L for one launch per wave, else the
  // whole device for each (one after the other)
  int conc = L > 1 && L <= kStackSlots;
  int rc = LSTM_ERR_UNSUPPORTED;
  for (int pass = conc ? 0 : 1; pass < 2; ++pass) {
    const int div = pass == 0 ? L : 1;
    rc = make_plan(T, shape->B, shape->I, shape->H, shape->dtype, &sp->pl[0], div);
    if (rc == LSTM_OK) rc = make_plan(T, shape->B, shape->H, shape->H, shape->dtype, &sp->pl[1], div);
    if (rc == LSTM_OK) {
      conc = pass == 0;
      break;
    }
    if (rc != LSTM_ERR_UNSUPPORTED) return rc;
  }
  if (rc != LSTM_OK) return rc;
  for (int i = 0; i < 2; ++i) {
    sp->pl[i].ijfo = (shape->flags & LSTM_GATES_IJFO) ? 1 : 0;
    sp->pl[i].two_bias = (shape->flags & LSTM_TWO_BIAS) ? 1 : 0;
  }
  sp->L = L;
  sp->C = C;
  sp->Tc = (int)Tc;
  sp->concurrent = conc;
  // block layout: the one-layer regions up to its cell record, then the
  // split-K partials (the larger of the whole-T and the chunk products), db
  // partials of every chunk, the layer's output and output cotangent, and
  // the fp32 carries of the chunks
  const Plan& a = sp->pl[0];
  const Plan& b = sp->pl[1];
  size_t region = a.off_gp > b.off_gp ? a.off_gp : b.off_gp;  // ctrl .. C of either layer kind
  size_t gp = 0;
  for (int i = 0; i < 2; ++i) {
    const size_t g0 = gemm_partial_bytes(sp->pl[i], sp->pl[i].cus);
    const size_t g1 = gemm_partial_bytes(chunk_of(sp->pl[i], Tc), sp->pl[i].cus);
    const size_t g2 = T > 0 ? gemm_partial_bytes(chunk_of(sp->pl[i], T - (int64_t)(C - 1) * Tc), sp->pl[i].cus) : 0;
    if (g0 > gp) gp = g0;
    if (g1 > gp) gp = g1;
    if (g2 > gp) gp = g2;
  }
  const int e = a.esize;
  sp->off_gp = region;
  sp->off_dbp = sp->off_gp + al256(gp);
  sp->off_y = sp->off_dbp + al256((size_t)C * a.nBG * a.G4 * 4);
  sp->off_dy = sp->off_y + al256((size_t)a.TB * a.H * e);
  sp->off_carry = sp->off_dy + al256((size_t)a.TB * a.H * e);
  const size_t block = sp->off_carry + al256((size_t)2 * a.B * a.H * 4);
  for (int l = 0; l <= L; ++l) sp->off_block[l] = (size_t)l * block;
  sp->total = (size_t)L * block;
  return LSTM_OK;
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
  if (concurrent) *concurrent = sp.concurrent;
  return LSTM_OK;
}

int lstm_stack_fwd_train(const lstm_shape* shape, int64_t layers, int64_t chunks, const void* x, const void* W,
                         const void* b, const void* h0, const void* c0, void* y, void* hT, void* cT, void* workspace,
                         size_t workspace_bytes, void* stream) {
  StackPlan sp;
  const int rc = stack_plan(shape, layers, chunks, &sp);
  if (rc != LSTM_OK) return rc;
  const Plan& p0 = sp.pl[0];
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
  if (B == 0) return LSTM_OK;
  const int64_t sst = B * H * e;
  if (T == 0) {
    err = launch_copy_state(h0, hT, (size_t)(L * B * H), e, s);
    if (err == hipSuccess) err = launch_copy_state(c0, cT, (size_t)(L * B * H), e, s);
    return status_from(err);
  }
  // per layer: its plan, weights, input and output
  auto plan_of = [&](int l) -> const Plan& { return sp.pl[l == 0 ? 0 : 1]; };
  auto wof = [&](int l) -> const char* {
    return (const char*)W + (l == 0 ? 0 : (G4 * (H + I) + (int64_t)(l - 1) * G4 * 2 * H) * e);
  };
  const int64_t bst = (p0.two_bias ? 2 : 1) * G4 * e;
  auto blk = [&](int l) { return ws + sp.off_block[l]; };
  auto yof = [&](int l) -> char* { return l == L - 1 ? (char*)y : blk(l) + sp.off_y; };
  auto xof = [&](int l) -> const char* { return l == 0 ? (const char*)x : yof(l - 1); };
  auto at = [](const void* q, int64_t off) -> const char* { return q ? (const char*)q + off : nullptr; };
  uint32_t* errw = (uint32_t*)(blk(0) + p0.off_ctrl);

  for (int w = 0; w < sp.C + L - 1 && err == hipSuccess; ++w) {
    FwdSlot sl[kMaxLayers];
    int ns = 0;
    for (int l = 0; l < L && err == hipSuccess; ++l) {
      const int k = w - l;
      if (k < 0 || k >= sp.C) continue;
      const Plan& pf = plan_of(l);
      const int64_t t0 = (int64_t)k * sp.Tc, tc = (T - t0) < sp.Tc ? (T - t0) : sp.Tc;
      const int64_t Il = l == 0 ? I : H;
      char* bl = blk(l);
      // the input projection of the chunk; its launch clears the layer's
      // exchange regions (and, first of all, the error word)
      const size_t z0 = (w == 0 && l == 0) ? pf.off_ctrl : pf.off_HX;
      Timed tm(0, s);
      err = launch_gemm_inproj(chunk_of(pf, tc), xof(l) + t0 * B * Il * e, wof(l), at(b, l * bst),
                               (float*)(bl + pf.off_P) + t0 * B * G4, (float*)(bl + sp.off_gp), bl + z0,
                               pf.off_PX + pf.bytes_PX - z0, s);
      sl[ns++] = FwdSlot{(const float*)(bl + pf.off_P) + t0 * B * G4,
                         wof(l),
                         H + Il,
                         k == 0 ? at(h0, l * sst) : yof(l) + (t0 - 1) * B * H * e,
                         k == 0 ? at(c0, l * sst) : nullptr,
                         k == 0 ? nullptr : (const float*)(bl + pf.off_C) + (t0 - 1) * B * H,
                         yof(l) + t0 * B * H * e,
                         (char*)hT + l * sst,
                         (char*)cT + l * sst,
                         bl + pf.off_G + t0 * B * G4 * e,
                         (float*)(bl + pf.off_C) + t0 * B * H,
                         (uint64_t*)(bl + pf.off_HX),
                         (int)tc,
                         0};
    }
    if (err != hipSuccess) break;
    // the wave's recurrences (plans of layers 0 and >= 1 share the layout)
    const Plan& pr = sp.pl[1];
    if (sp.concurrent) {
      Timed tm(1, s);
      err = launch_fwd_recurrent(pr, sl, ns, errw, nullptr, nullptr, s);
    } else {
      for (int i = 0; i < ns && err == hipSuccess; ++i) {
        Timed tm(1, s);
        err = launch_fwd_recurrent(pr, &sl[i], 1, errw, nullptr, nullptr, s);
      }
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
  const Plan& p0 = sp.pl[0];
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
  auto plan_of = [&](int l) -> const Plan& { return sp.pl[l == 0 ? 0 : 1]; };
  auto woff = [&](int l) -> int64_t { return l == 0 ? 0 : (G4 * (H + I) + (int64_t)(l - 1) * G4 * 2 * H) * e; };
  auto blk = [&](int l) { return ws + sp.off_block[l]; };
  auto yof = [&](int l) -> const char* { return l == L - 1 ? (const char*)y : blk(l) + sp.off_y; };
  auto xof = [&](int l) -> const char* { return l == 0 ? (const char*)x : yof(l - 1); };
  // output cotangent of layer l: the user's for the last layer, else the
  // input gradient of the layer above
  auto dyof = [&](int l) -> char* { return l == L - 1 ? (char*)dy : blk(l) + sp.off_dy; };
  auto at = [](const void* q, int64_t off) -> const char* { return q ? (const char*)q + off : nullptr; };
  uint32_t* errw = (uint32_t*)(blk(0) + p0.off_ctrl);

  for (int w = 0; w < sp.C + L - 1 && err == hipSuccess; ++w) {
    BwdSlot sl[kMaxLayers];
    int lay[kMaxLayers], chk[kMaxLayers];
    int ns = 0;
    for (int l = L - 1; l >= 0; --l) {
      const int k = (sp.C - 1) - (w - (L - 1 - l));
      if (k < 0 || k >= sp.C) continue;
      const Plan& pf = plan_of(l);
      const int64_t t0 = (int64_t)k * sp.Tc, tc = (T - t0) < sp.Tc ? (T - t0) : sp.Tc;
      char* bl = blk(l);
      lay[ns] = l;
      chk[ns] = k;
      sl[ns++] = BwdSlot{(const char*)W + woff(l),
                         H + (l == 0 ? I : H),
                         k == 0 ? at(c0, l * sst) : nullptr,
                         k == 0 ? nullptr : (const float*)(bl + pf.off_C) + (t0 - 1) * B * H,
                         dyof(l) + t0 * B * H * e,
                         k == sp.C - 1 ? at(dhT, l * sst) : nullptr,
                         k == sp.C - 1 ? at(dcT, l * sst) : nullptr,
                         bl + pf.off_G + t0 * B * G4 * e,
                         (const float*)(bl + pf.off_C) + t0 * B * H,
                         bl + pf.off_P + t0 * B * G4 * e,
                         (uint64_t*)(bl + pf.off_PX),
                         db ? (float*)(bl + sp.off_dbp) + (int64_t)k * pf.nBG * G4 : nullptr,
                         (char*)dh0 + l * sst,
                         (char*)dc0 + l * sst,
                         (float*)(bl + sp.off_carry),
                         k < sp.C - 1 ? 1 : 0,
                         k > 0 ? 1 : 0,
                         (int)tc,
                         0};
    }
    const Plan& pr = sp.pl[1];
    if (sp.concurrent) {
      Timed tm(2, s);
      err = launch_bwd_recurrent(pr, sl, ns, errw, nullptr, nullptr, s);
    } else {
      for (int i = 0; i < ns && err == hipSuccess; ++i) {
        Timed tm(2, s);
        err = launch_bwd_recurrent(pr, &sl[i], 1, errw, nullptr, nullptr, s);
      }
    }
    // each chunk's input gradient (the output cotangent of the layer below,
    // or dx), and its exchange cleared for the next chunk
    for (int i = 0; i < ns && err == hipSuccess; ++i) {
      const int l = lay[i], k = chk[i];
      const Plan& pf = plan_of(l);
      const int64_t t0 = (int64_t)k * sp.Tc, tc = (T - t0) < sp.Tc ? (T - t0) : sp.Tc;
      const int64_t Il = l == 0 ? I : H;
      char* bl = blk(l);
      Timed tm(4, s);
      if (Il > 0) {
        void* out = l == 0 ? (void*)((char*)dx + t0 * B * I * e) : (void*)(dyof(l - 1) + t0 * B * H * e);
        err = launch_gemm_dx(chunk_of(pf, tc), bl + pf.off_P + t0 * B * G4 * e, (const char*)W + woff(l), out,
                             (float*)(bl + sp.off_gp), nullptr, 0, s);
      }
      if (err == hipSuccess) err = launch_fill_zero(bl + pf.off_PX, pf.bytes_PX, s);
    }
  }
  // dW and db of each layer over all T*B rows
  for (int l = 0; l < L && err == hipSuccess; ++l) {
    Plan pf = plan_of(l);
    pf.dbp_rows = sp.C * pf.nBG;
    char* bl = blk(l);
    Timed tm(3, s);
    err = launch_gemm_dw(pf, bl + pf.off_P, xof(l), at(h0, l * sst), yof(l), (char*)dW + woff(l),
                         (float*)(bl + sp.off_gp), nullptr, 0, (const float*)(bl + sp.off_dbp),
                         db ? (char*)db + l * bst : nullptr, s);
  }
  return status_from(err);
}

}  // extern "C"
