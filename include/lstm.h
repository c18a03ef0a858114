/*
 * lstm.h -- C ABI of liblstm.so: forward pass and backpropagation through
 * time of a single-layer, unidirectional LSTM on one AMD Instinct MI355X
 * (gfx950), written in HIP.
 *
 * What is computed (the "SingleLayerLstmGrad" operator page, Ascend CANN
 * ops-nn: forward-formula table "前向传播公式" and the backward recursion
 * "反向传播算法" steps 1-6):
 *
 *   z_t = [h_{t-1}; x_t]                    h_{-1} = h0, c_{-1} = c0
 *   i,f,o = sigmoid(W_{i,f,o} z_t + b),     g = tanh(W_g z_t + b)
 *   c_t = f*c_{t-1} + i*g,                  h_t = o*tanh(c_t) = y_t
 *
 * and, given the cotangents dy (of every h_t), dhT (of the last h) and dcT
 * (of the last c), the exact gradients dx, dW, db, dh0, dc0 of the scalar
 * sum_t <dy_t,h_t> + <dhT,h_{T-1}> + <dcT,c_{T-1}>, by the page's step-by-
 * step recursion (the forget gate enters the cell carry once, as its cell-
 * gradient derivation requires).
 *
 * Layouts (all dense, row-major, time-major as in the page's parameter
 * table):
 *   x  [T,B,I]      y, dy [T,B,H]      h0, c0, hT, cT, dhT, dcT, dh0, dc0 [B,H]
 *   W  [4H, H+I]    row block k (rows [kH,(k+1)H)) is gate LSTM_GATE_* = k,
 *                   i.e. order i, f, g, o ("ifjo", j being the candidate g);
 *                   columns [0,H) multiply h_{t-1}, columns [H,H+I) multiply
 *                   x_t (the order of z_t)
 *   b, db [4H]      same gate order (the page's db shape [4,H] is the same
 *                   memory)
 *   dW [4H, H+I]
 * Element type: all of the above are LSTM_F32 (float) or all LSTM_BF16
 * (bfloat16 storage).  Every dot product accumulates in fp32; the cell state
 * is carried in fp32.
 *
 * Ownership and execution: the caller allocates every buffer (device
 * memory).  The library never allocates device memory, keeps no pointer
 * after a call returns, and launches asynchronously on the given stream
 * (a hipStream_t passed as void*; NULL = the default stream) without any
 * host synchronisation.  Buffers must stay alive until the stream has
 * drained.  Outputs are overwritten, never accumulated into.
 *
 * Workspace: opaque device memory of lstm_query() bytes, 256-byte aligned.
 * lstm_fwd_train() writes the forward record into it (activated gates and
 * cell states of every step -- the page's i/j/f/o/c inputs of the backward
 * operator); lstm_bwd() reads that record and must see it unmodified.
 * lstm_bwd() does not destroy the record, so it may be repeated.  Calls that
 * share one workspace must not overlap in time.
 *
 * Errors: every entry point returns LSTM_OK (0) or a negative LSTM_ERR_*
 * code.  All argument checks happen before any launch; on error nothing is
 * launched and no output is touched.  No C++ exception crosses the ABI.
 */
#ifndef LAYER_LSTM_AMD_LSTM_H
#define LAYER_LSTM_AMD_LSTM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LSTM_ABI_VERSION 2

/* Gate row blocks of W, b, dW, db (the "ifjo" order of the page's
 * gate_order attribute; LSTM_GATES_IJFO below selects "ijfo"). */
enum { LSTM_GATE_I = 0, LSTM_GATE_F = 1, LSTM_GATE_G = 2, LSTM_GATE_O = 3 };

/* Element type of every ABI tensor. */
enum { LSTM_F32 = 0, LSTM_BF16 = 1 };

/* Status codes. */
enum {
  LSTM_OK = 0,
  LSTM_ERR_NULL = -1,        /* a required pointer is NULL */
  LSTM_ERR_DIMS = -2,        /* T, B or I < 0, or H <= 0 */
  LSTM_ERR_DTYPE = -3,       /* dtype is not LSTM_F32 / LSTM_BF16, or an unknown flag is set */
  LSTM_ERR_ALIGN = -4,       /* a tensor is not aligned to its element size, or the workspace to 256 B */
  LSTM_ERR_WORKSPACE = -5,   /* workspace_bytes < lstm_query() */
  LSTM_ERR_UNSUPPORTED = -6, /* shape outside the kernels' envelope (see lstm_query) */
  LSTM_ERR_COOP = -7,        /* the persistent grid cannot be co-resident on this device */
  LSTM_ERR_LAUNCH = -8,      /* a HIP launch failed */
  LSTM_ERR_TIMEOUT = -9,     /* a per-step wait of the recurrent kernels hit its time bound */
  LSTM_ERR_DEVICE = -10      /* the current device is not gfx950 or could not be queried */
};

/* Direction of time (SingleLayerLstmGrad, 参数说明: the direction attribute,
 * forward or reverse).  The reverse direction runs the same cell from
 * t = T-1 down to t = 0: the step at time t reads h and c of time t+1, h0
 * and c0 enter at t = T-1, and hT / cT are the states after the step at
 * t = 0; dh0 / dc0 are the gradients of h0 / c0 as they enter.  Tensors
 * keep their [T][B][...] layout in both directions. */
enum { LSTM_REVERSE = 1 };

/* Gate order of W's, b's, dW's and db's row blocks (SingleLayerLstmGrad,
 * 参数说明: the gate_order attribute, "ifjo" or "ijfo").  Without this flag
 * the blocks are i, f, g, o (LSTM_GATE_I..O below, "ifjo"); with it they
 * are i, g, f, o ("ijfo", j being the candidate g).  The arithmetic is the
 * same; only the row blocks are relabelled. */
enum { LSTM_GATES_IJFO = 2 };

/* Two biases (bias_ih and bias_hh of the LSTMCell of the CMU 10-414 HW4 page): with this flag
 * b is [2][4H], the input-side bias then the hidden-side one, and the cell
 * adds both; db, when given, is [2][4H] and receives the bias gradient in
 * both halves (the two enter the pre-activation alike). */
enum { LSTM_TWO_BIAS = 4 };

/* Problem shape.  dtype is LSTM_F32 or LSTM_BF16; flags is 0 or an OR of
 * LSTM_REVERSE, LSTM_GATES_IJFO and LSTM_TWO_BIAS, other bits must be 0
 * (else LSTM_ERR_DTYPE).  The forward call and the backward call of one
 * record take the same flags. */
typedef struct {
  int64_t T; /* time steps, >= 0 */
  int64_t B; /* batch, >= 0 */
  int64_t I; /* input size, >= 0 */
  int64_t H; /* hidden size, >= 1 */
  int32_t dtype;
  int32_t flags; /* an OR of LSTM_REVERSE, LSTM_GATES_IJFO, LSTM_TWO_BIAS, or 0 */
} lstm_shape;

/* LSTM_ABI_VERSION of the library. */
int lstm_abi_version(void);

/* Human-readable text of a status code (static storage; never NULL). */
const char* lstm_status_string(int status);

/* Workspace size in bytes for `shape` on the current device.
 * Envelope: H <= 1024 (fp32) or 2048 (bf16), I <= 65536, T*B <= 2^31/4H,
 * T <= 2^30.  Returns LSTM_OK and sets
 * *workspace_bytes, or an error code (workspace_bytes untouched). */
int lstm_query(const lstm_shape* shape, size_t* workspace_bytes);

/* How the persistent recurrences are laid out for `shape` on the current
 * device, for measurement and reporting (the same choice lstm_fwd_train()
 * and lstm_bwd() make).  Work-group (bg, jg) of the grid owns batch rows
 * [bg*rows_per_group, +rows_per_group) and hidden units [jg*units_per_group,
 * +units_per_group).  A *_valu field is 1 when that recurrence runs its
 * product on the vector ALUs (fp32, 4-row groups) and 0 when it runs on the
 * matrix cores.  Returns LSTM_OK and fills *info, or an error code of
 * lstm_query() (info untouched). */
typedef struct {
  int32_t rows_per_group;  /* NB */
  int32_t units_per_group; /* NJ */
  int32_t groups;          /* batch groups (nBG) */
  int32_t units_groups;    /* work-groups per batch group (nJG) */
  int32_t grid;            /* work-groups of each recurrent launch */
  int32_t waves;           /* waves per work-group */
  int32_t xcd_local;       /* 1: every batch group runs on one XCD */
  int32_t fwd_valu;
  int32_t bwd_valu;
  int32_t inproj_tiles_per_wg; /* input projection: output tiles per work-group
                                  (> 1: persistent work-groups, one per CU;
                                  16-byte aligned x and W assumed) */
  int32_t reserved[6];
} lstm_plan_info;
int lstm_query_plan(const lstm_shape* shape, lstm_plan_info* info);

/* Forward pass for training ("前向传播公式").
 *   x [T,B,I], W [4H,H+I]: required (x may be NULL only if T*B*I == 0)
 *   b [4H], h0 [B,H], c0 [B,H]: optional, NULL = zero
 *   y [T,B,H], hT [B,H], cT [B,H]: outputs (y may be NULL only if T*B == 0)
 *   workspace: receives the forward record for lstm_bwd. */
int lstm_fwd_train(const lstm_shape* shape, const void* x, const void* W, const void* b,
                   const void* h0, const void* c0, void* y, void* hT, void* cT,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Backpropagation through time ("反向传播算法" steps 1-6).
 *   dy [T,B,H]: required; dhT, dcT [B,H]: optional, NULL = zero
 *   x, W, h0, c0, y: the same tensors the forward saw (h0 NULL = zero;
 *   c0 NULL = zero); the forward record in `workspace`
 *   dx [T,B,I], dW [4H,H+I], dh0 [B,H], dc0 [B,H]: outputs
 *   db [4H]: output, optional (NULL = not computed). */
int lstm_bwd(const lstm_shape* shape, const void* dy, const void* dhT, const void* dcT,
             const void* x, const void* W, const void* h0, const void* c0, const void* y,
             void* workspace, size_t workspace_bytes,
             void* dx, void* dW, void* db, void* dh0, void* dc0, void* stream);

/* Waits for `stream`, then reports (and clears) a time-out that a
 * recurrent kernel recorded in `workspace`: LSTM_ERR_TIMEOUT, else LSTM_OK
 * (or LSTM_ERR_LAUNCH if the stream itself reports an error).  The time-out
 * mark is set by the kernels themselves (a per-step wait that exceeded its
 * bound, e.g. because other work held the device's compute units for
 * seconds, or the device did not deal work-groups to its XCDs round robin
 * as the XCD-local layout relies on); it stays set, and the outputs of later calls on the workspace are
 * undefined, until lstm_fwd_train() runs again on it.  After any error,
 * run lstm_fwd_train() before the next lstm_bwd() on the same workspace. */
int lstm_check_workspace(void* workspace, size_t workspace_bytes, void* stream);

/* Per-kernel timing, for measurement.  While enabled (on != 0), every
 * kernel the library launches is bracketed by HIP events recorded on the
 * call's stream, and the elapsed time is added to the total of its kind:
 *   0 input projection   1 forward recurrence   2 backward recurrence
 *   3 dW product (with its split-K sum and the final db sum)   4 dx product
 *   5 (not used)   6 state copies of the T = 0 / B = 0 cases
 * lstm_timing_enable(1) also resets the totals.  lstm_timing_read() waits for
 * the recorded events and returns the total milliseconds and the launch
 * count of one kind.  Not thread-safe; timing adds a few microseconds per
 * launch. */
int lstm_timing_enable(int on);
int lstm_timing_read(int kind, double* total_ms, int64_t* launches);

/* Step-phase stamps of the recurrent kernels, for measurement.  With a
 * device buffer of at least 2*8*T*6 uint64 values set, each later call whose
 * sequence length is at most T makes thread 0 of work-groups 0..7 write the
 * 100 MHz real-time clock (s_memrealtime) at six points of every step:
 * forward -- step start, its h_{t-1} words read, all threads past the wait,
 * own product done, cross-wave sum done, outputs written; backward -- step
 * start, dh carry gathered, deltas written, partial products sent, next
 * operands requested, step end.  Layout: [pass (0 forward, 1 backward)]
 * [work-group][step in execution order][point].  NULL disables.  Returns
 * LSTM_ERR_WORKSPACE if the buffer is too small for T. */
int lstm_stamps_set(void* device_buffer, size_t bytes, int64_t T);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* LAYER_LSTM_AMD_LSTM_H */
