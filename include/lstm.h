/*
 * lstm.h -- C ABI of liblstm.so: forward pass and backpropagation through
 * time of a single-layer LSTM (one direction of time, either one, or both:
 * LSTM_BIDIRECTIONAL) on one AMD Instinct MI355X (gfx950), written in HIP.
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
 * Element type: all of the above are LSTM_F32 (float), all LSTM_BF16
 * (bfloat16 storage) or all LSTM_F16 (IEEE binary16 storage).  Every dot
 * product accumulates in fp32; the cell state is carried in fp32.
 *
 * Ownership and execution: the caller allocates every buffer (device
 * memory).  The library never allocates device memory, keeps no pointer
 * after a call returns, and launches asynchronously on the given stream
 * (a hipStream_t passed as void*; NULL = the default stream) without any
 * host synchronisation.  Buffers must stay alive until the stream has
 * drained.  Outputs are overwritten, never accumulated into.  Calls may be
 * issued on several streams: the persistent recurrent kernels (each holds
 * every compute unit it uses until its last step) of one device are
 * ordered by the library -- a launch on another stream than the previous
 * one first waits for that one -- so two of them never compete for the
 * compute units; the other kernels overlap freely.
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

#define LSTM_ABI_VERSION 3

/* Gate row blocks of W, b, dW, db (the "ifjo" order of the page's
 * gate_order attribute; LSTM_GATES_IJFO below selects "ijfo"). */
enum { LSTM_GATE_I = 0, LSTM_GATE_F = 1, LSTM_GATE_G = 2, LSTM_GATE_O = 3 };

/* Element type of every ABI tensor: fp32, or 16-bit storage -- bfloat16 or
 * IEEE binary16 (the FLOAT16 of the page's dtype column) -- with fp32
 * accumulation. */
enum { LSTM_F32 = 0, LSTM_BF16 = 1, LSTM_F16 = 2 };

/* Status codes. */
enum {
  LSTM_OK = 0,
  LSTM_ERR_NULL = -1,        /* a required pointer is NULL */
  LSTM_ERR_DIMS = -2,        /* T, B or I < 0, or H <= 0 */
  LSTM_ERR_DTYPE = -3,       /* dtype is not LSTM_F32 / LSTM_BF16 / LSTM_F16, or an unknown flag is set */
  LSTM_ERR_ALIGN = -4,       /* a tensor is not aligned to its element size, or the workspace to 256 B */
  LSTM_ERR_WORKSPACE = -5,   /* workspace_bytes < lstm_query() */
  LSTM_ERR_UNSUPPORTED = -6, /* shape outside the kernels' envelope (see lstm_query) */
  LSTM_ERR_COOP = -7,        /* the persistent grid cannot be co-resident on this device */
  LSTM_ERR_LAUNCH = -8,      /* a HIP launch failed */
  LSTM_ERR_TIMEOUT = -9,     /* a per-step wait of the recurrent kernels hit its time bound */
  LSTM_ERR_DEVICE = -10,     /* the current device is not gfx950 or could not be queried */
  LSTM_ERR_SCRATCH = -11,    /* lstm_fwd_train_scratch: the shape needs more than LSTM_SCRATCH_BYTES */
  LSTM_ERR_PLACEMENT = -12,  /* lstm_check_workspace: two work-groups of a recurrent launch took one
                                role (the device dealt them to its XCDs otherwise than the XCD-local
                                layout assumes); later calls on this device use the spread layout */
  LSTM_ERR_STATE = -13       /* lstm_check_workspace: the workspace's status word holds bits no call
                                writes (a workspace that no forward pass has filled) */
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

/* Bidirectional layer (the bidirectional recurrent layer of the PyTorch
 * recurrent-layer page; num_directions = 2): direction 0 runs forward in
 * time and direction 1 in reverse, each with its own weights and initial
 * state, on the same x.  With this flag
 *   W, dW [2][4H][H+I]    b, db [2][4H] (or [2][2][4H] with LSTM_TWO_BIAS)
 *   h0, c0, hT, cT, dhT, dcT, dh0, dc0 [2][B][H]   (direction-major)
 *   y, dy [T][B][2H]      (h_t of direction 0, then of direction 1)
 *   x, dx [T][B][I]       (dx: the sum of both directions' input gradients)
 * Not combinable with LSTM_REVERSE (else LSTM_ERR_DTYPE).  The two
 * recurrences run in one launch on half the compute units each when the
 * shape's layout fits that, else one after the other
 * (lstm_plan_info.directions_concurrent). */
enum { LSTM_BIDIRECTIONAL = 8 };

/* Problem shape.  dtype is LSTM_F32, LSTM_BF16 or LSTM_F16; flags is 0 or an
 * OR of LSTM_REVERSE, LSTM_GATES_IJFO, LSTM_TWO_BIAS and LSTM_BIDIRECTIONAL,
 * other bits must be 0 (else LSTM_ERR_DTYPE).  The forward call and the
 * backward call of one record take the same flags. */
typedef struct {
  int64_t T; /* time steps, >= 0 */
  int64_t B; /* batch, >= 0 */
  int64_t I; /* input size, >= 0 */
  int64_t H; /* hidden size, >= 1 */
  int32_t dtype;
  int32_t flags; /* an OR of the LSTM_REVERSE .. LSTM_BIDIRECTIONAL flags, or 0 */
} lstm_shape;

/* LSTM_ABI_VERSION of the library. */
int lstm_abi_version(void);

/* Human-readable text of a status code (static storage; never NULL). */
const char* lstm_status_string(int status);

/* Workspace size in bytes for `shape` on the current device.
 * Envelope: I <= 65536, T*B <= 2^31/4H, T <= 2^30, and a layout of the
 * persistent recurrences for B and H (their work-groups hold W_h in
 * registers, one per CU).  On a 256-CU MI355X: fp32 up to H = 512 (B up to
 * 256 at H = 512, more below), H = 640..1024 for B <= 8; 16-bit storage up to
 * H = 1024 (B up to 256 at H = 1024, more below), H up to 2048 for B <= 32
 * (64 at some sizes).  Outside it: LSTM_ERR_UNSUPPORTED.  Returns LSTM_OK and
 * sets *workspace_bytes, or an error code (workspace_bytes untouched). */
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
  int32_t directions_concurrent; /* LSTM_BIDIRECTIONAL: 1 when both recurrences
                                    run in one launch (grid above is per direction) */
  int32_t fwd_tagged;      /* 1: the forward recurrence exchanges h as tagged
                              words (two values and the step in 8 bytes,
                              polled in place) instead of a packed ring and
                              step flags (spread layout, 16-bit storage) */
  int32_t reserved[4];
} lstm_plan_info;
int lstm_query_plan(const lstm_shape* shape, lstm_plan_info* info);

/* seq_length (SingleLayerLstmGrad, 参数说明: the optional mask matrix
 * [T, Batch, hidden_size] for the actual length of each sequence), taken in
 * its per-sequence form: a device array of B int32 lengths, or NULL (every
 * step of every sequence is real).  Length L_b stands for the mask that is 1
 * at the steps t < L_b of sequence b and 0 past them.  A step with mask 0
 * holds the state: c_t = c_{t-1} and h_t = h_{t-1} (y_t = h_t repeats it),
 * so a sequence's final state is that after its last real step (in the
 * reverse direction its steps past L_b come first and leave h0, c0 as they
 * are), and such a step gets no gate deltas: its dy reaches the held state
 * unchanged.  Lengths are not clamped: L_b >= T is a full sequence, L_b <= 0
 * an empty one.  The forward and the backward of one record take the same
 * lengths. */

/* Forward pass for training ("前向传播公式").
 *   x [T,B,I], W [4H,H+I]: required (x may be NULL only if T*B*I == 0)
 *   b [4H], h0 [B,H], c0 [B,H]: optional, NULL = zero
 *   seq_length [B] int32: optional (see above; 4-byte aligned)
 *   y [T,B,H], hT [B,H], cT [B,H]: outputs (y may be NULL only if T*B == 0)
 *   workspace: receives the forward record for lstm_bwd. */
int lstm_fwd_train(const lstm_shape* shape, const void* x, const void* W, const void* b,
                   const void* h0, const void* c0, const void* seq_length, void* y, void* hT, void* cT,
                   void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * forward pass of lstm_fwd_train() with the library's own device array as
 * its workspace, so that the caller passes only inputs and outputs.  The
 * array holds LSTM_SCRATCH_BYTES per device; it is set up on the first call
 * on each device (its address looked up once, the device's ordering event
 * created) and kept until the process ends.  No call allocates memory.
 *   Arguments and results as lstm_fwd_train() without the workspace; the
 *   forward record stays in the array until the next call on the device
 *   (there is no matching backward: a training step uses lstm_fwd_train()).
 *   LSTM_ERR_SCRATCH (nothing launched, outputs untouched) when
 *   lstm_query() of the shape exceeds LSTM_SCRATCH_BYTES.
 * Every call on a device shares its array: calls that overlap in time on
 * one device (on different streams, or from several threads) race and give
 * undefined results; calls on one stream are safe.  A per-step time-out
 * leaves the outputs undefined and is not reported (the array is not the
 * caller's to inspect). */
#define LSTM_SCRATCH_BYTES (64u << 20)
int lstm_fwd_train_scratch(const lstm_shape* shape, const void* x, const void* W, const void* b,
                           const void* h0, const void* c0, const void* seq_length, void* y, void* hT,
                           void* cT, void* stream);

/* Backpropagation through time ("反向传播算法" steps 1-6).
 *   dy [T,B,H]: required; dhT, dcT [B,H]: optional, NULL = zero
 *   x, W, h0, c0, seq_length, y: the same tensors the forward saw (h0 NULL =
 *   zero; c0 NULL = zero); the forward record in `workspace`
 *   dx [T,B,I], dW [4H,H+I], dh0 [B,H], dc0 [B,H]: outputs
 *   db [4H]: output, optional (NULL = not computed). */
int lstm_bwd(const lstm_shape* shape, const void* dy, const void* dhT, const void* dcT,
             const void* x, const void* W, const void* h0, const void* c0, const void* seq_length,
             const void* y, void* workspace, size_t workspace_bytes,
             void* dx, void* dW, void* db, void* dh0, void* dc0, void* stream);

/* Waits for `stream`, then reports (and clears) a time-out that a
 * recurrent kernel recorded in `workspace`: LSTM_ERR_PLACEMENT when a launch
 * found two of its work-groups in one role (it then also timed out; later
 * plans on this device use the spread layout, see lstm_query_plan's
 * xcd_local), else LSTM_ERR_TIMEOUT, else LSTM_OK (or LSTM_ERR_LAUNCH if the
 * stream itself reports an error).  The time-out
 * mark is set by the kernels themselves (a per-step wait that exceeded its
 * bound, e.g. because other work held the device's compute units for
 * seconds, or the device did not deal work-groups to its XCDs round robin
 * as the XCD-local layout relies on); it stays set, and the outputs of later calls on the workspace are
 * undefined, until lstm_fwd_train() runs again on it.  After any error,
 * run lstm_fwd_train() before the next lstm_bwd() on the same workspace.
 * Every lstm_fwd_train() (T = 0 and B = 0 included) defines the status word;
 * a word with bits no call writes (a workspace no forward pass has filled)
 * gives LSTM_ERR_STATE and changes no layout choice. */
int lstm_check_workspace(void* workspace, size_t workspace_bytes, void* stream);

/* Per-kernel timing, for measurement.  While enabled (on != 0), every
 * kernel the library launches is bracketed by HIP events recorded on the
 * call's stream, and the elapsed time is added to the total of its kind:
 *   0 input projection   1 forward recurrence   2 backward recurrence
 *   3 dW product (with its split-K sum and the final db sum)   4 dx product
 *   5 direction copies (LSTM_BIDIRECTIONAL: y joined, dy split)
 *   6 state copies of the T = 0 / B = 0 cases
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

/* Stacked layers (the "Stack Multiple RNN Cells" of the MXNet LSTM page;
 * num_layers of the CMU 10-414 page's LSTM module): `layers` = L one-
 * direction layers, layer l + 1 taking layer l's output sequence as its
 * input; only the last layer's output is the stack's.  shape gives T, B, I
 * (layer 0's input size; the others' is H), H, the dtype, and flags 0 or
 * LSTM_GATES_IJFO / LSTM_TWO_BIAS (others: LSTM_ERR_DTYPE); 1 <= L <= 8.
 *   W, dW   the layers' weights back to back: layer 0 [4H][H+I], then layers
 *           1..L-1 [4H][2H] (columns [W_h | W_x] as above)
 *   b, db   [L][4H] (or [L][2][4H] with two biases); b may be NULL
 *   h0, c0, hT, cT, dhT, dcT, dh0, dc0   [L][B][H] (layer-major)
 *   x, dx   [T][B][I]      y, dy   [T][B][H] (the last layer's output)
 * Schedule (a wavefront): time is cut into `chunks` chunks (0: chunks of at
 * least 128 steps, at most 8 of them; chunks > T: T); in wave w layer l runs chunk w - l, so layer l + 1's steps of
 * chunk k run beside layer l's steps of chunk k + 1 -- in one persistent
 * launch per wave, each of its n layers on cus / n compute units, when the
 * recurrences have such a layout (n <= 4; *concurrent = the most layers one
 * launch runs, 1: one after the other).  A wave of one layer gives it the
 * whole device; chunks = 1 runs the layers one after the other.  Layer 0's
 * input projection and input gradient run once over all T.  The backward
 * runs the waves from the last chunk of the last layer down.  Results equal the layers run one after the other
 * (the state crosses chunk borders in fp32 as within a chunk).  Workspace,
 * errors, streams and ownership as for the one-layer calls; the forward and
 * the backward of one record take the same layers and chunks. */
int lstm_stack_query(const lstm_shape* shape, int64_t layers, int64_t chunks, size_t* workspace_bytes,
                     int32_t* concurrent);
int lstm_stack_fwd_train(const lstm_shape* shape, int64_t layers, int64_t chunks, const void* x, const void* W,
                         const void* b, const void* h0, const void* c0, void* y, void* hT, void* cT,
                         void* workspace, size_t workspace_bytes, void* stream);
int lstm_stack_bwd(const lstm_shape* shape, int64_t layers, int64_t chunks, const void* dy, const void* dhT,
                   const void* dcT, const void* x, const void* W, const void* h0, const void* c0, const void* y,
                   void* workspace, size_t workspace_bytes, void* dx, void* dW, void* db, void* dh0, void* dc0,
                   void* stream);

/* The floor under a recurrence step, for measurement: runs the forward
 * recurrence's per-step exchange alone -- the step flags of the batch group,
 * the copy of the group's h rows from the exchange ring into LDS, this
 * work-group's stores into the next ring slot and its flag -- for T steps,
 * in the layout lstm_fwd_train() uses for `shape` (layout 0), or that
 * layout with its batch groups spread over the XCDs (layout 1: device-
 * coherent stores, every exchange through memory), without the product or
 * the gate math.  `workspace` (lstm_query() bytes) is overwritten.  Runs the
 * probe once untimed, then once between two events; waits for the stream
 * and sets *us_per_step to the timed launch's time / T.  Returns
 * LSTM_OK, an error of lstm_query(), LSTM_ERR_DIMS (T or B < 1, or another
 * layout), or LSTM_ERR_TIMEOUT. */
int lstm_probe_exchange(const lstm_shape* shape, int layout, void* workspace, size_t workspace_bytes,
                        double* us_per_step, void* stream);

/* The parts of a stage of the pipelined bf16 products, for measurement:
 * runs one work-group of 8 waves (512 threads; two waves per SIMD, as the
 * products run) on every compute unit, each wave issuing `iters` iterations
 * of 32 v_mfma_f32_16x16x32_bf16 on operands in registers, plus the parts
 * of a product stage that `parts` (LSTM_PROBE_* bits) selects:
 *   LSTM_PROBE_READS        12 KB of fragment reads per wave from LDS,
 *                           before the iteration's products;
 *   LSTM_PROBE_READS_AHEAD  the same reads for the next iteration, issued
 *                           before this one's products (not with READS);
 *   LSTM_PROBE_BARRIER      one work-group barrier per iteration;
 *   LSTM_PROBE_DMA          four 1 KB direct-to-LDS loads per wave and
 *                           iteration from a 64 KB buffer, three iterations
 *                           in flight.
 * It computes nothing of the LSTM.  `scratch` is device memory of at least
 * LSTM_PROBE_SCRATCH_BYTES, 256-byte aligned, overwritten.  Runs the probe
 * once untimed, then once between two events; waits for the stream and sets
 * *frac_of_peak to the MFMA FLOPs / time / the dense bf16 peak (2516.6
 * TFLOP/s for 256 compute units, scaled to the device's count).  Returns
 * LSTM_OK, LSTM_ERR_NULL, LSTM_ERR_DIMS (unknown bits, both read orders, or
 * iters outside [1, 2^24]), LSTM_ERR_ALIGN, LSTM_ERR_WORKSPACE (scratch too
 * small), LSTM_ERR_DEVICE or LSTM_ERR_LAUNCH. */
enum { LSTM_PROBE_READS = 1, LSTM_PROBE_READS_AHEAD = 2, LSTM_PROBE_BARRIER = 4, LSTM_PROBE_DMA = 8 };
#define LSTM_PROBE_SCRATCH_BYTES ((size_t)1 << 20)
int lstm_probe_mfma_stage(int parts, int64_t iters, void* scratch, size_t scratch_bytes, double* frac_of_peak,
                          void* stream);

/* Test hooks, for the tests of the failure paths (host-side settings that
 * later calls copy into their launches; every kernel still exits normally):
 *   LSTM_DEBUG_FAIL_STEP, value s >= 0: at step s (in execution order) of
 *     every recurrent launch, work-group 0 records a time-out as if its wait
 *     had run past its bound; value < 0 turns this off;
 *   LSTM_DEBUG_MISPLACE, value 1: in the XCD-local layout, work-group 0 takes
 *     the role of the neighbouring XCD, as a device that dealt the
 *     work-groups differently would make it (two claimants of one role, one
 *     role empty: the launch times out and reports LSTM_ERR_PLACEMENT);
 *     0 turns this off;
 *   LSTM_DEBUG_XCD_LOCAL, value 1: allow the XCD-local layout on the current
 *     device again after LSTM_ERR_PLACEMENT (0: forbid it).
 * Returns LSTM_OK, or LSTM_ERR_DIMS for an unknown `what`.  Not thread-safe. */
enum { LSTM_DEBUG_FAIL_STEP = 1, LSTM_DEBUG_MISPLACE = 2, LSTM_DEBUG_XCD_LOCAL = 3 };
int lstm_debug_inject(int what, int64_t value);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* LAYER_LSTM_AMD_LSTM_H */
