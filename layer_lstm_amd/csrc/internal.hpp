// internal.hpp -- host-side plan and launcher declarations shared by the
// C-ABI layer and the kernel translation units (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lstm {

// Bit of the error word (first 4 bytes of the workspace) that a recurrent
// kernel sets when one of its per-step waits hits the time bound.
constexpr uint32_t kErrTimeout = 1u;
// Bit set (with kErrTimeout) when two work-groups of a launch took one role:
// the device did not deal the work-groups to its XCDs as the XCD-local
// layout assumes (one role then stays empty and its readers time out).
constexpr uint32_t kErrPlacement = 2u;

// Phase stamps of the recurrent kernels (see lstm_stamps_set in lstm.h).
constexpr int kStampWGs = 8, kPhases = 6;

// Work partition and workspace layout of one problem shape.
struct Plan {
  int64_t T, B, I, H;
  int dtype;   // 0 = fp32, 1 = bf16, 2 = fp16 (storage)
  int esize;   // bytes per storage element
  int64_t TB, G4, Z;  // T*B, 4H, H+I

  // persistent recurrent kernels: a grid of nBG x nJG work-groups; group
  // (bg, jg) owns batch rows [bg*NB, (bg+1)*NB) and hidden units
  // [jg*NJ, (jg+1)*NJ)
  int NB, NJ, nBG, nJG, grid;
  int Hp;       // H rounded up to a power of two (>= 4 MFMA k-blocks)
  int waves;    // waves per work-group of the MFMA recurrences (4 or 8)
  int fwd_nkbw; // forward: W_h k-blocks per wave
  int fwd_mw;   // forward: M-tiles per wave (1 or 2)
  int fwd_dma;  // forward: h ring copied by direct-to-LDS loads (rows of whole KB), split ring-read phase
  int fwd_tag;  // forward: h exchanged as tagged words, no step flags (spread layout; recurrent.hip)
  int bwd_mt;   // backward (MFMA): 16-unit tiles of W_h^T per work-group
  int bwd_nkb;  // backward (MFMA): k-blocks of the 4H gate rows per wave
  int bwd_valu; // backward runs the VALU kernel (fp32, batch groups of 4 rows)
  int words_per_thread;  // exchange words a thread reads per step (NB*H / 256, rounded up)
  int Bp;       // nBG * NB
  size_t lds_fwd, lds_bwd;
  // XCD-local exchange: when the batch groups divide evenly over the XCDs
  // (nBG a multiple of nxcd), each batch group lives on one XCD and its
  // exchange words stay in that XCD's L2 (plain stores, device-coherent
  // loads).
  int nxcd;     // XCDs of the device (compute units / 32 on gfx950)
  int xcd_local;

  // workspace (byte offsets, 256-aligned)
  size_t off_ctrl, off_P, off_G, off_C, off_HX, off_PX, off_dbp, total;
  size_t bytes_HX, bytes_PX;
  // flag exchange (MFMA kernels): packed payload at the start of the HX / PX
  // region (h ring, gate-delta ring), step flags at these byte offsets
  // inside it
  size_t off_hflags, off_pflags;
  // role claims of the persistent launches (one word per work-group role,
  // cleared with their exchange region): at these byte offsets inside HX
  // (forward) and PX (backward)
  size_t off_hclaim, off_pclaim;
  // test hooks (lstm_debug_inject): the step at which work-group 0 acts as
  // if its wait had timed out (-1: never), and work-group 0 reading the
  // wrong XCD in the XCD-local layout
  int fail_step, misplace;
  int rev;          // 1: the reverse direction (steps from t = T-1 down to 0)
  int ijfo;         // 1: W, b, dW, db in the gate order i, g, f, o (gate_block)
  int two_bias;     // 1: b and db are [2][4H] (b_ih, b_hh)
  // bidirectional layer: two direction blocks of dir_bytes each, holding
  // the one-direction layout above plus that direction's y and dy
  // ([T][B][H] at off_ydir, off_dydir inside the block), then the fp32 dx
  // sums [TB][I] at off_dxacc; concurrent: both recurrences in one launch
  // (the plan laid out for half the compute units each), else one after the
  // other
  int bidir, concurrent;
  size_t dir_bytes, off_ydir, off_dydir, off_dxacc;
  // rows of db partials the dW launch sums ([rows][4H]; 0: nBG, one set of
  // steps)
  int dbp_rows;
  int cus;          // compute units of the device
  int max_splits;   // largest split-K factor of the three products
  size_t off_gp;    // fp32 split-K partials of the products
};

// Brackets the launches made during its lifetime with two events on the
// stream when per-kernel timing is on (lstm_timing_enable), adding their
// elapsed time to the total of `kind`.
struct Timed {
  int kind;
  hipStream_t s;
  hipEvent_t a = nullptr;
  Timed(int k, hipStream_t st);
  ~Timed();
  Timed(const Timed&) = delete;
  Timed& operator=(const Timed&) = delete;
};

// LDS through which the MFMA recurrences gather their W_h slices at start.
constexpr size_t kColStageLds = 80 * 1024;

// Waves of the VALU recurrences and of the 4-wave MFMA ones.
constexpr int kWaves = 4;
constexpr int kRecThreads = 64 * kWaves;

// Fill the plan for a shape; returns 0 or an LSTM_ERR_* code.
// cap_div: the recurrences' grid may take cus / cap_div compute units.
int make_plan(int64_t T, int64_t B, int64_t I, int64_t H, int dtype, Plan* p, int cap_div = 1);

// The plan runs the VALU forward (fp32 batch groups of 4 rows).
bool fwd_vec_ok(const Plan& p);

// ---- launchers (return hipError_t) ----
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_copy_state(const void* src, void* dst, size_t n, int esize, hipStream_t s);

// The three products.  `part` holds the fp32 split-K partials (null = do not
// split); the launch also clears `zero_bytes` at `zero` (may be 0).
// P[tb][4j+g] = sum_k x[tb][k] W[gH+j][H+k] + b[gH+j]   (fp32 out)
hipError_t launch_gemm_inproj(const Plan& p, const void* x, const void* W, const void* b, float* P, float* part,
                              void* zero, size_t zero_bytes, hipStream_t s);
// dx[tb][i] = sum_n dG[tb][n] W[row(n)][H+i]; with acc_out the fp32 sums go
// there instead of dx, with acc_in they are added to it before the rounding
// to dx (the two directions of a bidirectional layer)
hipError_t launch_gemm_dx(const Plan& p, const void* dG, const void* W, void* dx, float* part, void* zero,
                          size_t zero_bytes, hipStream_t s, float* acc_out = nullptr, const float* acc_in = nullptr);
// dW[row(m)][n] = sum_tb dG[tb][m] Z[tb][n],  Z = [h_{t-1} | x_t]
// The dW launch also writes db[row(n)] = sum_bg DBP[bg][n] (in bg order) when
// db is not null.
hipError_t launch_gemm_dw(const Plan& p, const void* dG, const void* x, const void* h0, const void* y, void* dW,
                          float* part, void* zero, size_t zero_bytes, const float* DBP, void* db, hipStream_t s);
size_t gemm_partial_bytes(const Plan& p, int cus);
// output tiles per work-group of the input projection (1: one tile each;
// 16-byte aligned operands assumed)
int inproj_tiles_per_wg(const Plan& p);

// One recurrence of a persistent launch and its tensors.  A launch runs up
// to four (the two directions of a bidirectional layer, or the layers of a
// stack's wave), each on grid work-groups of the plan's layout.
struct FwdSlot {
  const float* P;   // [T][B][4H] fp32 input projection of the slot's steps
  const void* W;    // the layer's [4H][Z] weights (W_h = the first H columns)
  int64_t Z;        // W's row length: H plus the layer's input size
  const void* h0;   // [B][H] or null
  const void* c0;   // [B][H] or null
  const float* c0f; // [B][H] fp32 initial cell state in place of c0, or null
  void* y;          // [T][B][H]
  void* hT;         // [B][H]
  void* cT;         // [B][H]
  void* Gs;         // [T][B][4H] activated gates (record)
  float* Cs;        // [T][B][H] cell states (record)
  uint64_t* HX;     // the slot's exchange region (cleared before the launch)
  int T, rev;       // steps of the launch; direction of time
};
struct BwdSlot {
  const void* W;
  int64_t Z;
  const void* c0;       // [B][H] or null: c_{-1} of the first step
  const float* cprevf;  // fp32 c_{-1} of the first step in place of c0, or null
  const void* dy;       // [T][B][H]
  const void* dhT;      // [B][H] or null
  const void* dcT;      // [B][H] or null
  const void* Gs;
  const float* Cs;
  void* dG;             // [T][B][4H] gate deltas (record)
  uint64_t* PX;         // the slot's exchange region (cleared before the launch)
  float* DBP;           // [nBG][4H] db partials of the slot's steps, or null
  void* dh0;
  void* dc0;
  float* carry;         // [2][B][H] fp32 carries (dh, dc) or null
  int carry_in, carry_out;  // read the carries instead of dhT/dcT; write them instead of dh0/dc0
  int T, rev;
};

// The persistent recurrences of `nslots` slots in one launch of nslots x
// grid work-groups (every slot on the plan's layout); len: [B] sequence
// lengths or null; err: the error word every slot reports to.
hipError_t launch_fwd_recurrent(const Plan& p, const FwdSlot* slots, int nslots, uint32_t* err, uint64_t* stamps,
                                const int32_t* len, hipStream_t s);
hipError_t launch_bwd_recurrent(const Plan& p, const BwdSlot* slots, int nslots, uint32_t* err, uint64_t* stamps,
                                const int32_t* len, hipStream_t s);
// The forward recurrence's exchange alone (exchange_probe.hip): flags, ring
// copy, ring stores, no arithmetic; HX must start cleared.
hipError_t launch_exchange_probe(const Plan& p, void* HX, uint32_t* err, hipStream_t s);
// The parts of a stage of the pipelined bf16 products (mfma_probe.hip):
// `parts` of the kProbe* bits (LSTM_PROBE_* of lstm.h), at most one of the
// two read orders; grid work-groups of 512 threads; src: 64 KB, sink: grid
// x 512 floats.
constexpr int kProbeReads = 1, kProbeReadsAhead = 2, kProbeBarrier = 4, kProbeDma = 8;
hipError_t launch_mfma_probe(int parts, int grid, const uint32_t* src, float* sink, int iters, hipStream_t s);
// The two directions' [rows][H] outputs side by side into [rows][2H]
// (join), or [rows][2H] cotangents back into two [rows][H] (split).
hipError_t launch_join_dirs(const void* y0, const void* y1, void* y, int64_t rows, int64_t row_bytes, hipStream_t s);
hipError_t launch_split_dirs(const void* dy, void* dy0, void* dy1, int64_t rows, int64_t row_bytes, hipStream_t s);

}  // namespace lstm
