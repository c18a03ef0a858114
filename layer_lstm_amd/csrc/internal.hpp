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

// Phase stamps of the recurrent kernels (see lstm_stamps_set in lstm.h).
constexpr int kStampWGs = 8, kPhases = 6;

// Work partition and workspace layout of one problem shape.
struct Plan {
  int64_t T, B, I, H;
  int dtype;   // 0 = fp32, 1 = bf16
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
  int rev;          // 1: the reverse direction (steps from t = T-1 down to 0)
  int ijfo;         // 1: W, b, dW, db in the gate order i, g, f, o (gate_block)
  int two_bias;     // 1: b and db are [2][4H] (b_ih, b_hh)
  int cus;          // compute units of the device
  int max_splits;   // largest split-K factor of the three products
  size_t off_gp;    // fp32 split-K partials of the products
};

// LDS through which the MFMA recurrences gather their W_h slices at start.
constexpr size_t kColStageLds = 80 * 1024;

// Waves of the VALU recurrences and of the 4-wave MFMA ones.
constexpr int kWaves = 4;
constexpr int kRecThreads = 64 * kWaves;

// Fill the plan for a shape; returns 0 or an LSTM_ERR_* code.
int make_plan(int64_t T, int64_t B, int64_t I, int64_t H, int dtype, Plan* p);

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
// dx[tb][i] = sum_n dG[tb][n] W[row(n)][H+i]
hipError_t launch_gemm_dx(const Plan& p, const void* dG, const void* W, void* dx, float* part, void* zero,
                          size_t zero_bytes, hipStream_t s);
// dW[row(m)][n] = sum_tb dG[tb][m] Z[tb][n],  Z = [h_{t-1} | x_t]
// The dW launch also writes db[row(n)] = sum_bg DBP[bg][n] (in bg order) when
// db is not null.
hipError_t launch_gemm_dw(const Plan& p, const void* dG, const void* x, const void* h0, const void* y, void* dW,
                          float* part, void* zero, size_t zero_bytes, const float* DBP, void* db, hipStream_t s);
size_t gemm_partial_bytes(const Plan& p, int cus);
// output tiles per work-group of the input projection (1: one tile each;
// 16-byte aligned operands assumed)
int inproj_tiles_per_wg(const Plan& p);

hipError_t launch_fwd_recurrent(const Plan& p, const float* P, const void* W, const void* h0,
                                const void* c0, void* y, void* hT, void* cT, void* Gs, float* Cs,
                                uint64_t* HX, uint32_t* err, uint64_t* stamps, hipStream_t s);
hipError_t launch_bwd_recurrent(const Plan& p, const void* W, const void* c0, const void* dy,
                                const void* dhT, const void* dcT, const void* Gs, const float* Cs,
                                void* dG, uint64_t* PX, float* DBP, void* dh0, void* dc0, uint32_t* err,
                                uint64_t* stamps, hipStream_t s);

}  // namespace lstm
