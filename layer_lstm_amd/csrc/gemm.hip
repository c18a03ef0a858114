// gemm.hip -- MFMA GEMMs of the LSTM path (gfx950) and the small helpers.
//
// One tiled core serves the three products of the method:
//   input projection  P  = X  . W_x^T + b   (M=T*B, N=4H, K=I)
//   input gradient    dX = dG . W_x         (M=T*B, N=I,  K=4H)
//   weight gradient   dW = dG^T . Z         (M=4H,  N=H+I, K=T*B), Z=[h_{t-1}|x_t]
// ("SingleLayerLstmGrad" page: pre-activations W z_t + b of the forward
// table; parameter gradient sum_t delta_t z_t^T of step 4; delta-z = W^T
// delta of step 5, whose input block is dx.)
//
// Gate rows are handled in an interleaved order inside the path: column
// n = 4j + g of P / dG is gate g of hidden unit j (row gH + j of W), so that
// the recurrent kernels find the four gates of one unit next to each other.
//
// Tiles: 128 x 128 (or 64 x 64 when 128-wide tiles would leave compute units
// idle) per 256-thread work-group, 4 waves in 2 x 2, 128 bytes of k per
// stage (32 fp32 or 64 bf16 / fp16), double-buffered in LDS; K is split when even
// the smaller tiles cannot give every compute unit a tile.
// Both operands sit in LDS as [row][k] with a 16-byte row pad; an operand
// whose contiguous dimension is M or N is transposed in registers on its way
// into LDS.  Accumulation is fp32 (v_mfma_f32_16x16x4f32 for fp32 storage,
// v_mfma_f32_16x16x32_bf16 / _f16 for bf16 / fp16 storage).  Split-K partials are summed
// by a second kernel in a fixed order, so results are run-to-run identical.
#include "device_common.hpp"
#include "internal.hpp"

namespace lstm {

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;            // k bytes per stage and row
constexpr int kLdsRow = kRowBytes + 16;   // padded LDS row

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

__device__ __forceinline__ int64_t gate_row(int64_t n, int64_t H, int ijfo) {
  return (int64_t)gate_block((int)(n & 3), ijfo) * H + (n >> 2);
}

// ---------------------------------------------------------------------------
// Operand accessors.  VEC = elements per 16 bytes.
//
// KRows: element (r, k) at row_ptr(r)[k] (k contiguous).
// MNRows: element (k, r) at krow_ptr(k)[r] (r contiguous).
template <typename T>
struct KRowsX {  // plain row-major [R][ld], rows r, k in [0,K)
  const T* p; int64_t ld; int64_t R, K; bool vec_ok;
  __device__ __forceinline__ const T* row(int64_t r) const { return p + r * ld; }
};
template <typename T>
struct KRowsWx {  // row r (interleaved gate row) of W's input block
  const T* W; int64_t H, ld, R, K; bool vec_ok; int ijfo;
  __device__ __forceinline__ const T* row(int64_t r) const { return W + gate_row(r, H, ijfo) * ld + H; }
};
template <typename T>
struct MNRowsWx {  // k-row = interleaved gate row of W's input block, r = input column
  const T* W; int64_t H, ld, R, K; bool vec_ok; int ijfo;
  __device__ __forceinline__ const T* krow(int64_t k, int64_t r) const { return W + gate_row(k, H, ijfo) * ld + H + r; }
  __device__ __forceinline__ bool same_seg(int64_t, int64_t) const { return true; }
};
template <typename T>
struct MNRowsPlain {  // [K][ld], r contiguous
  const T* p; int64_t ld, R, K; bool vec_ok;
  __device__ __forceinline__ const T* krow(int64_t k, int64_t r) const { return p + k * ld + r; }
  __device__ __forceinline__ bool same_seg(int64_t, int64_t) const { return true; }
};
template <typename T>
struct MNRowsZ {  // Z[tb][r] = r < H ? h_prev(t)[b][r] : x[tb][r-H]
  // h_prev(t): the hidden state the step at time t read -- y[t-1] (h0 at
  // t = 0), or y[t+1] (h0 at t = T-1) in the reverse direction (rev)
  const T* x; const T* h0; const T* y; int64_t B, H, I, R, K; bool vec_ok; bool rev;
  __device__ __forceinline__ const T* krow(int64_t tb, int64_t r) const {
    if (r < H) {
      if (!rev && tb >= B) return y + (tb - B) * H + r;
      if (rev && tb < K - B) return y + (tb + B) * H + r;
      const int64_t b = rev ? tb - (K - B) : tb;
      return h0 ? h0 + b * H + r : nullptr;  // nullptr = zero initial state
    }
    return x + tb * I + (r - H);
  }
  // r..r+n-1 do not straddle the h/x boundary
  __device__ __forceinline__ bool same_seg(int64_t r, int64_t n) const { return (r >= H) || (r + n <= H); }
};

template <typename T>
__device__ __forceinline__ u32x4_t load_krow_vec(const T* rowp, int64_t k, int64_t K, bool vec_ok) {
  constexpr int VEC = 16 / sizeof(T);
  u32x4_t v = {0, 0, 0, 0};
  if (rowp == nullptr) return v;
  if (vec_ok && k + VEC <= K) {
    v = *reinterpret_cast<const u32x4_t*>(rowp + k);
  } else {
    T tmp[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) tmp[i] = (k + i < K) ? rowp[k + i] : T(0);
    v = __builtin_bit_cast(u32x4_t, tmp);
  }
  return v;
}

// 16 bytes along r at fixed k; zero outside [0,R) x [0,K)
template <typename T, class Op>
__device__ __forceinline__ u32x4_t load_mn_vec(const Op& op, int64_t k, int64_t r) {
  constexpr int VEC = 16 / sizeof(T);
  u32x4_t v = {0, 0, 0, 0};
  if (k >= op.K || r >= op.R) return v;
  if (op.vec_ok && r + VEC <= op.R && op.same_seg(r, VEC)) {
    const T* p = op.krow(k, r);
    if (p) v = *reinterpret_cast<const u32x4_t*>(p);
    return v;
  }
  T tmp[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    T e = T(0);
    if (r + i < op.R) {
      const T* p = op.krow(k, r + i);
      if (p) e = *p;
    }
    tmp[i] = e;
  }
  return __builtin_bit_cast(u32x4_t, tmp);
}

// ---------------------------------------------------------------------------
// Stage loaders: fetch one ROWS x (128 bytes of k) tile into registers, then
// write it to LDS as [row][k].
template <int ROWS, typename T, class Op, bool MN>
struct Stager;

// k-contiguous source: ROWS rows x 8 vectors, ROWS/32 per thread
template <int ROWS, typename T, class Op>
struct Stager<ROWS, T, Op, false> {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int NV = ROWS * 8 / kThreads;
  u32x4_t v[NV];
  __device__ __forceinline__ void fetch(const Op& op, int64_t row0, int64_t k0, int tid) {
#pragma unroll
    for (int s = 0; s < NV; ++s) {
      const int id = tid + s * kThreads;
      const int r = id >> 3, kv = id & 7;
      const int64_t gr = row0 + r;
      v[s] = (gr < op.R) ? load_krow_vec<T>(op.row(gr), k0 + kv * VEC, op.K, op.vec_ok) : u32x4_t{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int s = 0; s < NV; ++s) {
      const int id = tid + s * kThreads;
      const int r = id >> 3, kv = id & 7;
      *reinterpret_cast<u32x4_t*>(lds + r * kLdsRow + kv * 16) = v[s];
    }
  }
};

// r-contiguous source: blocks of 2 k-rows x (16 bytes of r), ROWS/64 per
// thread; transposed into pairs (k, k+1) per r
template <int ROWS, typename T, class Op>
struct Stager<ROWS, T, Op, true> {
  static constexpr int VEC = 16 / sizeof(T);                // r per vector
  static constexpr int KPAIRS = kRowBytes / sizeof(T) / 2;  // k pairs per stage
  static constexpr int NB = ROWS * 4 / kThreads;            // blocks per thread
  u32x4_t v0[NB], v1[NB];
  __device__ __forceinline__ void fetch(const Op& op, int64_t row0, int64_t k0, int tid) {
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      const int id = tid + s * kThreads;
      const int rv = id / KPAIRS, kp = id % KPAIRS;
      const int64_t k = k0 + 2 * kp, r = row0 + rv * VEC;
      v0[s] = load_mn_vec<T>(op, k, r);
      v1[s] = load_mn_vec<T>(op, k + 1, r);
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      const int id = tid + s * kThreads;
      const int rv = id / KPAIRS, kp = id % KPAIRS;
      const T* a = reinterpret_cast<const T*>(&v0[s]);
      const T* b = reinterpret_cast<const T*>(&v1[s]);
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        T pair[2] = {a[i], b[i]};
        char* dst = lds + (rv * VEC + i) * kLdsRow + kp * 2 * (int)sizeof(T);
        if constexpr (sizeof(T) == 2)
          *reinterpret_cast<uint32_t*>(dst) = __builtin_bit_cast(uint32_t, pair);
        else
          *reinterpret_cast<uint64_t*>(dst) = __builtin_bit_cast(uint64_t, pair);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Epilogues: called once per output element (m < M, n < N) with the full
// dot product (after the split-K sum when the product is split).
// store4(m, n, v): the four outputs (m, n..n+3) at once, n a multiple of 4
// with n + 3 < N and the row start 16-byte (fp32) / 8-byte (bf16) aligned.
__device__ __forceinline__ void store_row4(bf16_t* p, f32x4_t v) {
  const uint32_t lo = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  const uint32_t hi = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
  *(uint2*)p = uint2{lo, hi};
}
__device__ __forceinline__ void store_row4(f16_t* p, f32x4_t v) {
  const f16_t h[4] = {(f16_t)v[0], (f16_t)v[1], (f16_t)v[2], (f16_t)v[3]};
  *(uint2*)p = __builtin_bit_cast(uint2, h);
}
__device__ __forceinline__ void store_row4(float* p, f32x4_t v) { *(f32x4_t*)p = v; }

struct EpiP {  // fp32 P with bias in the interleaved column order
  // (two: the bias is the sum of two [4H] vectors, bias[r] + bias[ldp + r])
  float* P; const void* bias; int64_t H, ldp; int dtype; int ijfo; int two;
  __device__ __forceinline__ float bias_at(int64_t n) const {
    const int64_t r = gate_row(n, H, ijfo);
    float v = load_as_f(bias, r, dtype);
    if (two) v += load_as_f(bias, ldp + r, dtype);
    return v;
  }
  __device__ __forceinline__ void operator()(int64_t m, int64_t n, float v) const {
    if (bias) v += bias_at(n);
    P[m * ldp + n] = v;
  }
  // column term of columns n..n+3 (the bias), added by the caller of store4
  __device__ __forceinline__ f32x4_t col4(int64_t n) const {
    if (!bias) return f32x4_t{0.f, 0.f, 0.f, 0.f};
    return f32x4_t{bias_at(n), bias_at(n + 1), bias_at(n + 2), bias_at(n + 3)};
  }
  __device__ __forceinline__ void store4(int64_t m, int64_t n, f32x4_t v) const { store_row4(P + m * ldp + n, v); }
};
template <typename T>
struct EpiStore {  // plain row-major output of the storage type
  T* out; int64_t ld;
  __device__ __forceinline__ void operator()(int64_t m, int64_t n, float v) const {
    out[m * ld + n] = Elem<T>::from_f(v);
  }
  __device__ __forceinline__ f32x4_t col4(int64_t) const { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ void store4(int64_t m, int64_t n, f32x4_t v) const { store_row4(out + m * ld + n, v); }
};
template <typename T>
struct EpiAdd {  // out = storage(prev + v): the second of two products summed in fp32
  T* out; const float* prev; int64_t ld;
  __device__ __forceinline__ void operator()(int64_t m, int64_t n, float v) const {
    out[m * ld + n] = Elem<T>::from_f(prev[m * ld + n] + v);
  }
  __device__ __forceinline__ f32x4_t col4(int64_t) const { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ void store4(int64_t m, int64_t n, f32x4_t v) const {
    store_row4(out + m * ld + n, v + *(const f32x4_t*)(prev + m * ld + n));
  }
};
template <typename T>
struct EpiDW {  // dW rows back in gate-block order
  T* dW; int64_t H, N; int ijfo;
  __device__ __forceinline__ void operator()(int64_t m, int64_t n, float v) const {
    dW[gate_row(m, H, ijfo) * N + n] = Elem<T>::from_f(v);
  }
  __device__ __forceinline__ f32x4_t col4(int64_t) const { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ void store4(int64_t m, int64_t n, f32x4_t v) const {
    store_row4(dW + gate_row(m, H, ijfo) * N + n, v);
  }
};

template <class AOp, class BOp, class Epi>
struct GemmArgs {
  int64_t M, N, K;
  int ktiles_per_split, splits;
  AOp a;
  BOp b;
  Epi epi;
  float* part;        // [splits][M][N] fp32 partial products when splits > 1
  uint32_t* zero;     // extra duty: clear `zero_words` words here (may be null)
  int64_t zero_words;
  const float* dsum;  // extra duty: dsum_out[row(n)] = sum_r dsum[r][n] (r < dsum_rows)
  void* dsum_out;     // (null = none); row(n) = gate-block order, storage dtype dsum_dtype
  int dsum_rows;
  int dsum_dtype;     // 0 fp32, 1 bf16, 2 fp16
  int64_t dsum_cols, dsum_H;
  int dsum_ijfo;      // gate-block order of dsum_out (gate_block)
  int dsum_two;       // dsum_out is [2][dsum_cols]: the sums written to both halves
  int nxcd;           // XCDs of the device (1: no XCD-aware tile order)
  // persistent input projection (gemm_lds_multi_kernel) only:
  int tiles_x, tiles_y;  // output tiles along n and m
  int per_wg;            // output tiles per work-group
};

// Output tile (n tile, m tile, split) of this work-group.  The device deals
// the work-groups of a dispatch to its XCDs round robin (from a starting XCD
// that varies), so work-groups i and i + nxcd share an XCD and its L2.  Each
// residue class mod nxcd is given one contiguous range of the row-major
// tile order (n fastest, then m, then split): the tiles an XCD runs at once
// then share rows of A and columns of B in its L2, instead of every XCD
// streaming every row-block of A.  Products with few tiles per split keep
// the plain order (there an XCD would work one K slice with all its CUs).
struct TileId {
  int64_t x, y;
  int z;
};
__device__ __forceinline__ TileId tile_of(int nxcd, int splits) {
  const int64_t gx = gridDim.x, gxy = (int64_t)gridDim.x * gridDim.y;
  const int64_t nc = gxy * splits;
  int64_t i = ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gx + blockIdx.x;
  if (nxcd > 1 && nc % nxcd == 0 && gxy >= 8 * nxcd) i = (i % nxcd) * (nc / nxcd) + i / nxcd;
  TileId t;
  t.z = (int)(i / gxy);
  const int64_t r = i - t.z * gxy;
  t.y = r / gx;
  t.x = r - t.y * gx;
  return t;
}

// ---------------------------------------------------------------------------
// Tile BM x BN = (32*WM) x (32*WN): 4 waves in 2 x 2, each (16*WM) x (16*WN).
// grid = (N tiles, M tiles, splits [+ 1 slab of clearing blocks]).
template <typename T, int WM, int WN, class AOp, bool AMN, class BOp, bool BMN, class Epi>
__global__ void __launch_bounds__(kThreads) gemm_kernel(GemmArgs<AOp, BOp, Epi> g) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int BM = 32 * WM, BN = 32 * WN;
  constexpr int ATILE = BM * kLdsRow, BTILE = BN * kLdsRow;
  char* As = smem;                 // [2][BM][kLdsRow]
  char* Bs = smem + 2 * ATILE;     // [2][BN][kLdsRow]
  constexpr int KSTAGE = kRowBytes / sizeof(T);  // k elements per stage

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if ((int)blockIdx.z == g.splits) {  // extra duties: clearing, db sum
    const int64_t nblk = (int64_t)gridDim.x * gridDim.y;
    const int64_t blk = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    for (int64_t i = blk * kThreads + tid; i < g.zero_words; i += nblk * kThreads) g.zero[i] = 0u;
    if (g.dsum_out) {
      for (int64_t n = blk * kThreads + tid; n < g.dsum_cols; n += nblk * kThreads) {
        float v = 0.f;
        for (int r = 0; r < g.dsum_rows; ++r) v += g.dsum[(int64_t)r * g.dsum_cols + n];
        const int64_t row = gate_row(n, g.dsum_H, g.dsum_ijfo);
        for (int h = 0; h <= g.dsum_two; ++h) {
          const int64_t o = row + h * g.dsum_cols;
          store_from_f(g.dsum_out, o, v, g.dsum_dtype);
        }
      }
    }
    return;
  }
  const int wm = w >> 1, wn = w & 1;
  const TileId tl = tile_of(g.nxcd, g.splits);
  const int64_t m0 = tl.y * BM, n0 = tl.x * BN;
  const int split = tl.z;
  const int64_t ktiles = (g.K + KSTAGE - 1) / KSTAGE;
  const int64_t kt_begin = (int64_t)split * g.ktiles_per_split;
  const int64_t kt_end = kt_begin + g.ktiles_per_split < ktiles ? kt_begin + g.ktiles_per_split : ktiles;

  f32x4_t acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  Stager<BM, T, AOp, AMN> sa;
  Stager<BN, T, BOp, BMN> sb;
  if (kt_begin < kt_end) {
    sa.fetch(g.a, m0, kt_begin * KSTAGE, tid);
    sb.fetch(g.b, n0, kt_begin * KSTAGE, tid);
    sa.store(As, tid);
    sb.store(Bs, tid);
  }
  __syncthreads();

  const int fr = lane & 15, fq = lane >> 4;
  for (int64_t kt = kt_begin; kt < kt_end; ++kt) {
    const int st = (int)((kt - kt_begin) & 1);
    const bool more = kt + 1 < kt_end;
    if (more) {
      sa.fetch(g.a, m0, (kt + 1) * KSTAGE, tid);
      sb.fetch(g.b, n0, (kt + 1) * KSTAGE, tid);
    }
    const char* a_st = As + st * ATILE + (wm * 16 * WM + fr) * kLdsRow + fq * 16;
    const char* b_st = Bs + st * BTILE + (wn * 16 * WN + fr) * kLdsRow + fq * 16;
#pragma unroll
    for (int kb = 0; kb < kRowBytes / 64; ++kb) {
      u32x4_t af[WM], bfv[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) af[i] = *reinterpret_cast<const u32x4_t*>(a_st + i * 16 * kLdsRow + kb * 64);
#pragma unroll
      for (int j = 0; j < WN; ++j) bfv[j] = *reinterpret_cast<const u32x4_t*>(b_st + j * 16 * kLdsRow + kb * 64);
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = Mfma<T>::mac(af[i], bfv[j], acc[i][j]);
    }
    if (more) {
      sa.store(As + (st ^ 1) * ATILE, tid);
      sb.store(Bs + (st ^ 1) * BTILE, tid);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int64_t n = n0 + wn * 16 * WN + j * 16 + fr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t m = m0 + wm * 16 * WM + i * 16 + fq * 4 + e;
        if (m < g.M && n < g.N) {
          if (g.splits > 1)
            g.part[((int64_t)split * g.M + m) * g.N + n] = acc[i][j][e];
          else
            g.epi(m, n, acc[i][j][e]);
        }
      }
    }
}

// ---------------------------------------------------------------------------
// Pipelined products (K a multiple of one stage): every operand is loaded
// straight into LDS (buffer_load_dwordx4 ... lds, no register staging) through a
// ring of kStages stages -- four stages of loads in flight while one is
// multiplied (the bf16 ring fills the 160 KB of LDS) -- in stages of 64
// bytes of k per tile row:
//   bf16: 256 x 256 tiles, 8 waves (2 x 4 of 128 x 64, two per SIMD), 32 k
//         per stage; the large tile halves the bytes loaded per MFMA against
//         128 x 128 tiles, which is what bounds those (the vector memory
//         path, not the MFMA);
//   fp32: 128 x 128 tiles, 4 waves (2 x 2 of 64 x 64), 16 k per stage (the
//         fp32 MFMA needs 16 times fewer bytes per cycle).
// Both shapes give 512-byte k-rows for r-contiguous operands and two loads
// per wave per operand and stage.
//   k-contiguous operand (rows of 64 bytes per stage): 16-byte chunk c of
//     tile row r sits at position c ^ krow_swz(r), so the rows of an MFMA
//     fragment read spread over the banks;
//   r-contiguous operand (512-byte k-rows): chunk c of k-row kr sits at
//     position c ^ mnrow_swz(kr); a fragment (16 rows x 16 bytes of
//     consecutive k per lane) is assembled from this [k][r] layout -- bf16:
//     two ds_read_b64_tr_b16, lane L of each 16-lane group pointing at
//     k-row kb + L/4, columns 4*(L%4)..+3, and receiving row L's four k
//     values; fp32: four 4-byte reads -- so both layouts feed the same
//     fragments.
// Tile rows or columns past the operand are loaded from its last valid rows
// (their outputs are never stored); an absent operand block (zero initial
// state) is read through an empty buffer descriptor, which returns zeros.
constexpr int kStages = 5;
static_assert(kStages == 5, "the stage waits in gemm_lds_kernel assume a 5-stage ring");

template <typename T> struct LdsCfg;
template <> struct LdsCfg<bf16_t> {
  static constexpr int kTile = 256, kWaves = 8, kThreads = 512, kKStage = 32;
};
template <> struct LdsCfg<f16_t> {
  static constexpr int kTile = 256, kWaves = 8, kThreads = 512, kKStage = 32;
};
template <> struct LdsCfg<float> {
  static constexpr int kTile = 128, kWaves = 4, kThreads = 256, kKStage = 16;
};
template <typename T> constexpr int lds_stage_bytes() { return 2 * LdsCfg<T>::kTile * 64; }

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Chunk swizzles.  k-contiguous tile (64-byte rows, 4 chunks): rows that an
// MFMA fragment read puts in one LDS pass -- 8 consecutive rows of one
// parity, or 16 consecutive rows of one residue mod 4 -- get distinct chunk
// positions.  r-contiguous tile (512-byte k-rows): the 4 k-rows of a
// transposed-read lane group, and the two groups 8 k-rows apart, get
// distinct 32-byte positions.
__device__ __forceinline__ int krow_swz(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int mnrow_swz(int kr) { return ((kr & 3) | (((kr >> 3) & 1) << 2)) << 1; }

// Direct-to-LDS loaders with launch-constant lane offsets: each of a lane's
// two 16-byte loads per operand and stage reads one buffer at (a per-lane
// offset fixed for the launch) + (a per-stage offset, uniform), through
// lds_dma16 (the stage waits below are the only ones).  The buffers are
// below 2 GiB (checked on the host).  Rows (krows) or columns (mnrows) past
// the operand are clamped to its last valid ones (their outputs are never
// stored).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
// (lds: LDS byte address of the wave's kilobyte)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t vo, uint32_t so) {
  lds_dma16_at<false>(r, lds, vo, so);
}
template <typename T, class Op, bool MN> struct Dma;
template <typename T, class Op>
struct DmaKRows {  // k-contiguous rows: row(r) = base + (rowidx(r) * ld + col0) elements
  __amdgpu_buffer_rsrc_t r;
  uint32_t vo[2];
  template <class RowIdx>
  __device__ __forceinline__ void init(const T* base, int64_t rows_total, int64_t ld, int64_t col0, int64_t R,
                                       int64_t row0, int w, int lane, RowIdx rowidx) {
    constexpr int VEC = 16 / sizeof(T);
    r = rsrc_of(base, rows_total * ld * (int64_t)sizeof(T));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rr = 32 * w + 16 * j + (lane >> 2), c = (lane & 3) ^ krow_swz(rr);
      int64_t gr = row0 + rr;
      gr = gr < R ? gr : R - 1;
      vo[j] = (uint32_t)((rowidx(gr) * ld + col0 + c * VEC) * (int64_t)sizeof(T));
    }
  }
  __device__ __forceinline__ void issue(uint32_t lds, int64_t k0, int w, int) const {
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(r, lds + (32 * w + 16 * j) * 64, vo[j], (uint32_t)(k0 * (int64_t)sizeof(T)));
  }
};
template <typename T>
struct Dma<T, KRowsX<T>, false> : DmaKRows<T, KRowsX<T>> {
  __device__ __forceinline__ Dma(const KRowsX<T>& op, int64_t row0, int w, int lane) {
    this->init(op.p, op.R, op.ld, 0, op.R, row0, w, lane, [](int64_t g) { return g; });
  }
};
template <typename T>
struct Dma<T, KRowsWx<T>, false> : DmaKRows<T, KRowsWx<T>> {
  __device__ __forceinline__ Dma(const KRowsWx<T>& op, int64_t row0, int w, int lane) {
    const int64_t H = op.H;
    const int ijfo = op.ijfo;
    this->init(op.W, 4 * H, op.ld, H, op.R, row0, w, lane, [H, ijfo](int64_t g) { return gate_row(g, H, ijfo); });
  }
};
// r-contiguous k-rows: lane (kr, chunk c) of a stage, r = r0 + c * VEC
__device__ __forceinline__ int mn_kr(int w, int j, int lane) { return 4 * w + 2 * j + (lane >> 5); }
template <typename T>
__device__ __forceinline__ int64_t mn_r(int64_t r0, int64_t R, int kr, int lane) {
  constexpr int VEC = 16 / sizeof(T);
  const int c = (lane & 31) ^ mnrow_swz(kr);
  const int64_t r = r0 + c * VEC;
  return r + VEC <= R ? r : R - VEC;
}
template <typename T>
struct Dma<T, MNRowsPlain<T>, true> {  // [K][ld]
  __amdgpu_buffer_rsrc_t r;
  uint32_t vo[2];
  int64_t ldb;
  __device__ __forceinline__ Dma(const MNRowsPlain<T>& op, int64_t r0, int w, int lane) {
    r = rsrc_of(op.p, op.K * op.ld * (int64_t)sizeof(T));
    ldb = op.ld * (int64_t)sizeof(T);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kr = mn_kr(w, j, lane);
      vo[j] = (uint32_t)(kr * ldb + mn_r<T>(r0, op.R, kr, lane) * (int64_t)sizeof(T));
    }
  }
  __device__ __forceinline__ void issue(uint32_t lds, int64_t k0, int w, int) const {
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(r, lds + (4 * w + 2 * j) * 512, vo[j], (uint32_t)(k0 * ldb));
  }
};
template <typename T>
struct Dma<T, MNRowsWx<T>, true> {  // k-row = interleaved gate row of W's input block
  __amdgpu_buffer_rsrc_t r;
  uint32_t vo[2];
  int64_t ldb;
  __device__ __forceinline__ Dma(const MNRowsWx<T>& op, int64_t r0, int w, int lane) {
    r = rsrc_of(op.W, 4 * op.H * op.ld * (int64_t)sizeof(T));
    ldb = op.ld * (int64_t)sizeof(T);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kr = mn_kr(w, j, lane);  // stage k-rows start at a multiple of 4: gate kr & 3, unit + kr / 4
      vo[j] = (uint32_t)(((int64_t)gate_block(kr & 3, op.ijfo) * op.H + (kr >> 2)) * ldb +
                         (op.H + mn_r<T>(r0, op.R, kr, lane)) * (int64_t)sizeof(T));
    }
  }
  __device__ __forceinline__ void issue(uint32_t lds, int64_t k0, int w, int) const {
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(r, lds + (4 * w + 2 * j) * 512, vo[j], (uint32_t)((k0 >> 2) * ldb));
  }
};
template <typename T>
struct Dma<T, MNRowsZ<T>, true> {  // Z[tb] = [h_prev(t)[b] | x[tb]]
  // three buffers, all addressed as [tb][...] with the stage's first k-row
  // tb0 = k0 as the uniform offset: h0 for the rows tb in [hlo, hhi) -- the
  // first B rows, or the last B in the reverse direction -- (absent: an empty
  // buffer, read as zeros), y shifted by B rows (back, or forward in the
  // reverse direction) for the others, and x
  __amdgpu_buffer_rsrc_t rh, ry, rx;
  uint32_t vh[2], vx[2];
  bool seg[2];  // load j's columns lie in the h part (the swizzle moves a
                // lane's column chunk between its k-rows, across the h / x
                // border where H is not a multiple of 16 chunks)
  int64_t hlo, hhi, hb, ib;
  __device__ __forceinline__ Dma(const MNRowsZ<T>& op, int64_t r0, int w, int lane) {
    constexpr int64_t E = sizeof(T);
    hb = op.H * E;
    ib = op.I * E;
    hlo = op.rev ? op.K - op.B : 0;
    hhi = op.rev ? op.K : op.B;
    rh = op.h0 ? rsrc_of((const char*)op.h0 - hlo * hb, hhi * hb) : rsrc_of(op.x, 0);
    // only offsets of the y rows are read
    ry = op.rev ? rsrc_of((const char*)op.y + op.B * hb, (op.K - op.B) * hb)
                : rsrc_of((const char*)op.y - op.B * hb, op.K * hb);
    rx = rsrc_of(op.x, op.K * ib);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kr = mn_kr(w, j, lane);
      const int64_t rj = mn_r<T>(r0, op.R, kr, lane);
      seg[j] = rj < op.H;
      vh[j] = (uint32_t)(kr * hb + rj * E);
      vx[j] = (uint32_t)(kr * ib + (rj - op.H) * E);
    }
  }
  // The branches end in distinct empty asm statements: the compiler would
  // otherwise merge their loads into one with a per-lane descriptor, which
  // it can only issue in a loop over the lanes' values.
  __device__ __forceinline__ void issue(uint32_t lds, int64_t k0, int w, int lane) const {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t dst = lds + (4 * w + 2 * j) * 512;
      if (!seg[j]) {
        dma16(rx, dst, vx[j], (uint32_t)(k0 * ib));
        asm volatile("; z: x part" ::: "memory");
      } else if (k0 + mn_kr(w, j, lane) >= hlo && k0 + mn_kr(w, j, lane) < hhi) {
        dma16(rh, dst, vh[j], (uint32_t)(k0 * hb));
        asm volatile("; z: h0 part" ::: "memory");
      } else {
        dma16(ry, dst, vh[j], (uint32_t)(k0 * hb));
        asm volatile("; z: y part" ::: "memory");
      }
    }
  }
};

__device__ __forceinline__ u32x4_t frag_krows(const char* lds, int row, int c) {
  return *(const u32x4_t*)(lds + row * 64 + ((c ^ krow_swz(row)) << 4));
}

template <typename T>
__device__ __forceinline__ u32x4_t frag_mnrows(const char* lds, int rbase, int lane) {
  u32x4_t out;
  if constexpr (sizeof(T) == 2) {
    const int grp = lane >> 4, L = lane & 15;
    const int m = rbase + 4 * (L & 3), c = m >> 3;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int kr = 8 * grp + 4 * hh + (L >> 2);
      const char* p = lds + kr * 512 + ((c ^ mnrow_swz(kr)) << 4) + ((m & 7) << 1);
      const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
      const uint2 u = __builtin_bit_cast(uint2, v);
      out[2 * hh] = u.x;
      out[2 * hh + 1] = u.y;
    }
  } else {
    // lane (fr, fq): row rbase + fr, k = 4 fq + s for s = 0..3
    const int m = rbase + (lane & 15), c = m >> 2, fq = lane >> 4;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const int kr = 4 * fq + sl;
      out[sl] = *(const uint32_t*)(lds + kr * 512 + ((c ^ mnrow_swz(kr)) << 4) + ((m & 3) << 2));
    }
  }
  return out;
}

template <typename T, int AMN, int BMN, class AOp, class BOp, class Epi>
__global__ void __launch_bounds__(LdsCfg<T>::kThreads, 1) gemm_lds_kernel(GemmArgs<AOp, BOp, Epi> g) {
  constexpr int TILE = LdsCfg<T>::kTile, NT = LdsCfg<T>::kThreads, KST = LdsCfg<T>::kKStage;
  constexpr int STAGE = lds_stage_bytes<T>();
  __shared__ __attribute__((aligned(16))) char ring0[STAGE], ring1[STAGE], ring2[STAGE], ring3[STAGE], ring4[STAGE];
  constexpr int WGN = LdsCfg<T>::kWaves / 2;  // waves along n (2 along m)
  constexpr int WM = TILE / 2 / 16, WN = TILE / WGN / 16;
  // the wave index is uniform: saying so keeps the direct-to-LDS addresses in
  // scalar registers (a divergent one would be iterated over lane values)
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  if ((int)blockIdx.z == g.splits) {  // extra duties: clearing, db sum
    const int64_t nblk = (int64_t)gridDim.x * gridDim.y;
    const int64_t blk = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    for (int64_t i = blk * NT + tid; i < g.zero_words; i += nblk * NT) g.zero[i] = 0u;
    if (g.dsum_out) {
      for (int64_t n = blk * NT + tid; n < g.dsum_cols; n += nblk * NT) {
        float v = 0.f;
        for (int r = 0; r < g.dsum_rows; ++r) v += g.dsum[(int64_t)r * g.dsum_cols + n];
        const int64_t row = gate_row(n, g.dsum_H, g.dsum_ijfo);
        for (int h = 0; h <= g.dsum_two; ++h) {
          const int64_t o = row + h * g.dsum_cols;
          store_from_f(g.dsum_out, o, v, g.dsum_dtype);
        }
      }
    }
    return;
  }
  const int wm = w / WGN, wn = w % WGN, fr = lane & 15, fq = lane >> 4;
  const TileId tl = tile_of(g.nxcd, g.splits);
  const int64_t m0 = tl.y * TILE, n0 = tl.x * TILE;
  const int split = tl.z;
  const int64_t ktiles = g.K / KST;
  const int64_t kt_begin = (int64_t)split * g.ktiles_per_split;
  const int64_t kt_end = kt_begin + g.ktiles_per_split < ktiles ? kt_begin + g.ktiles_per_split : ktiles;

  const Dma<T, AOp, (bool)AMN> da(g.a, m0, w, lane);
  const Dma<T, BOp, (bool)BMN> db(g.b, n0, w, lane);
  // LDS byte addresses of the ring slots (taken from the arrays themselves)
  const uint32_t rl[kStages] = {(uint32_t)(uintptr_t)(lds_void_t*)ring0, (uint32_t)(uintptr_t)(lds_void_t*)ring1,
                                (uint32_t)(uintptr_t)(lds_void_t*)ring2, (uint32_t)(uintptr_t)(lds_void_t*)ring3,
                                (uint32_t)(uintptr_t)(lds_void_t*)ring4};
  auto issue = [&](int64_t kt, uint32_t st) {
    da.issue(st, kt * KST, w, lane);
    db.issue(st + STAGE / 2, kt * KST, w, lane);
  };

  f32x4_t acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // column terms of this lane's output columns, fetched while the tile runs
  f32x4_t colt[WN];
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const int64_t n = n0 + wn * 16 * WN + j * 16 + 4 * fq;
    colt[j] = (g.splits == 1 && (g.N & 3) == 0 && n + 3 < g.N) ? g.epi.col4(n) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Fragments of a stage and its products.  Every fragment of a stage is
  // read before the first product (a scheduling barrier keeps the compiler
  // from interleaving the reads with the products and waiting on each pair).
  u32x4_t bfv[WN], afv[WM];
  auto read_frags = [&](const char* cur) {
    const int ln = lane, lfr = fr, lfq = fq;
    const char* sa = cur;
    const char* sb = cur + STAGE / 2;
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      if constexpr (BMN) bfv[j] = frag_mnrows<T>(sb, wn * 16 * WN + 16 * j, ln);
      else bfv[j] = frag_krows(sb, wn * 16 * WN + 16 * j + lfr, lfq);
    }
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      if constexpr (AMN) afv[i] = frag_mnrows<T>(sa, wm * 16 * WM + 16 * i, ln);
      else afv[i] = frag_krows(sa, wm * 16 * WM + 16 * i + lfr, lfq);
    }
  };
  // B as the MFMA's first operand: the tile comes out transposed, lane
  // (fr, fq) holding C[m = .. + fr][n = .. + 4 fq + e], four consecutive
  // columns for one row -- one 16-byte store per tile
  auto products = [&]() {
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) acc[i][j] = Mfma<T>::mac(bfv[j], afv[i], acc[i][j]);
  };
  // With both operands read transposed (dW), the two waves of a SIMD
  // (waves w and w + 4: halves wm = 0 and 1 of the tile) run a stage in
  // opposite orders, so that one reads fragments while the other multiplies:
  // wm = 0 leads (the products of stage kt from fragments read in the step
  // before, then the fragments of stage kt + 1), wm = 1 follows (the
  // fragments of stage kt, then its products).  Every wave then waits for
  // stage kt + 1 in step kt, two stages of loads staying in flight instead
  // of three: dW 905 -> 873 us on the largest workload, while dx went from
  // 463 to 477 us, so the other products keep the plain order.
  constexpr bool kPingPong = AMN == 1;
  const bool lead = kPingPong && wm == 0;
  // One step (stage kt in `cur`, kt + 1 in `nextc`): the stage waited for
  // (kt + 1 with the ping-pong order, else kt) is complete once at most
  // (stages issued after it) x 4 loads of this wave are outstanding
  // (s_waitcnt immediate: vmcnt bits [3:0] and [15:14], expcnt and lgkmcnt
  // at their no-wait maxima); the barrier then covers the other waves -- a
  // bare barrier, since __syncthreads() would also wait for every load in
  // flight -- and also tells that every wave is done with `nxt` (the slot of
  // stage kt - 1), refilled with stage kt + 4.
  auto stage = [&](int64_t kt, const char* cur, const char* nextc, uint32_t nxt) {
    const int64_t after = kt_end - 1 - kt;
    if constexpr (kPingPong) {
      if (after >= kStages - 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));
      else if (after == 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
      else if (after == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    } else {
      if (after >= kStages - 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(12));
      else if (after == 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));
      else if (after == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    __builtin_amdgcn_s_barrier();
    if (kt + kStages - 1 < kt_end) issue(kt + kStages - 1, nxt);
    if (!lead) read_frags(cur);
    __builtin_amdgcn_sched_barrier(0);
    products();
    __builtin_amdgcn_sched_barrier(0);
    if (lead && after >= 1) read_frags(nextc);
    __builtin_amdgcn_sched_barrier(0);
  };

  if (kt_begin + 0 < kt_end) issue(kt_begin + 0, rl[0]);
  if (kt_begin + 1 < kt_end) issue(kt_begin + 1, rl[1]);
  if (kt_begin + 2 < kt_end) issue(kt_begin + 2, rl[2]);
  if (kt_begin + 3 < kt_end) issue(kt_begin + 3, rl[3]);
  if (kPingPong && kt_begin < kt_end) {
    // stage kt_begin complete everywhere; the leading waves read it
    const int64_t nk = kt_end - kt_begin;
    if (nk >= 4) __builtin_amdgcn_s_waitcnt(vmcnt_imm(12));
    else if (nk == 3) __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));
    else if (nk == 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_s_barrier();
    if (lead) read_frags(ring0);
  }
  int64_t kt = kt_begin;
  for (; kt + kStages - 1 < kt_end; kt += kStages) {
    stage(kt, ring0, ring1, rl[4]);
    stage(kt + 1, ring1, ring2, rl[0]);
    stage(kt + 2, ring2, ring3, rl[1]);
    stage(kt + 3, ring3, ring4, rl[2]);
    stage(kt + 4, ring4, ring0, rl[3]);
  }
  if (kt < kt_end) stage(kt, ring0, ring1, rl[4]);
  if (kt + 1 < kt_end) stage(kt + 1, ring1, ring2, rl[0]);
  if (kt + 2 < kt_end) stage(kt + 2, ring2, ring3, rl[1]);
  if (kt + 3 < kt_end) stage(kt + 3, ring3, ring4, rl[2]);

  const bool vec_n = (g.N & 3) == 0;
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int64_t m = m0 + wm * 16 * WM + i * 16 + fr;
      const int64_t n = n0 + wn * 16 * WN + j * 16 + 4 * fq;
      if (m >= g.M || n >= g.N) continue;
      if (vec_n && n + 3 < g.N) {
        if (g.splits > 1) *(f32x4_t*)(g.part + ((int64_t)split * g.M + m) * g.N + n) = acc[i][j];
        else g.epi.store4(m, n, acc[i][j] + colt[j]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (n + e >= g.N) break;
          if (g.splits > 1) g.part[((int64_t)split * g.M + m) * g.N + n + e] = acc[i][j][e];
          else g.epi(m, n + e, acc[i][j][e]);
        }
      }
    }
}

// value of lane (lane ^ 8): DPP rotation by 8 within each row of 16 lanes
__device__ __forceinline__ float lane_xor8(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
}

// Persistent form for products whose operands are both k-contiguous rows
// (the input projection): one work-group per CU walks per_wg output tiles,
// and its loads form one stream over them, so the first stages of a tile
// are in flight while the previous tile ends and writes its outputs.  Four
// ring slots, the stages per tile a multiple of four: every tile starts in
// slot 0 and its loop is unrolled over the ring.  splits == 1; a second
// slab of work-groups (blockIdx.z == 1) only clears `zero`.  The tiles of an
// XCD (work-groups i mod nxcd) are one contiguous range of the tile order,
// walked together, each work-group taking every (work-groups per XCD)-th;
// within the range the order runs over blocks of 4 x 8 tiles (tm, tn below).
template <typename T, class AOp, class BOp, class Epi>
__global__ void __launch_bounds__(LdsCfg<T>::kThreads, 1) gemm_lds_multi_kernel(GemmArgs<AOp, BOp, Epi> g) {
  constexpr int TILE = LdsCfg<T>::kTile, KST = LdsCfg<T>::kKStage;
  constexpr int STAGE = lds_stage_bytes<T>();
  constexpr int NS = 4;
  constexpr int kColTable = 8192;  // column terms held in LDS (floats): N <= 8192
  __shared__ __attribute__((aligned(16))) char ring[NS * STAGE];
  __shared__ __attribute__((aligned(16))) float coltab[kColTable];
  constexpr int WGN = LdsCfg<T>::kWaves / 2;  // waves along n (2 along m)
  constexpr int WM = TILE / 2 / 16, WN = TILE / WGN / 16;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (blockIdx.z == 1) {
    const int64_t nt = (int64_t)gridDim.x * LdsCfg<T>::kThreads;
    for (int64_t i = (int64_t)blockIdx.x * LdsCfg<T>::kThreads + tid; i < g.zero_words; i += nt) g.zero[i] = 0u;
    return;
  }
  // The column terms (the bias) of every output column go into LDS once,
  // before the stream of loads starts, when the columns come in fours and
  // fit: a tile then reads its terms from LDS, and no global load of them
  // sits between one tile's P stores and the next tile's stages.
  const bool ctab = (g.N & 3) == 0 && g.N <= kColTable;
  if (ctab) {
    for (int64_t n = 4 * (int64_t)tid; n < g.N; n += 4 * (int64_t)LdsCfg<T>::kThreads)
      *(f32x4_t*)(coltab + n) = g.epi.col4(n);
    __syncthreads();
  }
  const int wm = w / WGN, wn = w % WGN, fr = lane & 15, fq = lane >> 4;
  const int i = blockIdx.x, per_xcd = g.tiles_x * g.tiles_y / g.nxcd;
  // Tile t of an XCD's range in blocks of 4 row-tiles x 8 column-tiles (the
  // 32 tiles its work-groups run at once: 6 MB of operands at 256 x 256 x
  // 1024 against 10 MB for 2 whole tile rows), where the range holds whole
  // blocks; else row-major.
  const bool blk48 = per_xcd % g.tiles_x == 0 && (per_xcd / g.tiles_x) % 4 == 0 && g.tiles_x % 8 == 0;
  auto tm = [&](int t) -> int {
    if (!blk48) return t / g.tiles_x;
    const int r = t % per_xcd, bq = r >> 5, e = r & 31;
    return (t - r) / g.tiles_x + (bq / (g.tiles_x >> 3)) * 4 + (e >> 3);
  };
  auto tn = [&](int t) -> int {
    if (!blk48) return t % g.tiles_x;
    const int r = t % per_xcd, bq = r >> 5, e = r & 31;
    return (bq % (g.tiles_x >> 3)) * 8 + (e & 7);
  };
  const int tstep = (int)gridDim.x / g.nxcd;
  const int tile0 = (i % g.nxcd) * per_xcd + i / g.nxcd;
  const int nk = (int)(g.K / KST);  // stages per tile
  const int S = nk * g.per_wg;      // stages of the stream

  int it = tile0, ik = 0;  // tile and stage of the next load
  Dma<T, AOp, false> da(g.a, (int64_t)tm(it) * TILE, w, lane);
  Dma<T, BOp, false> db(g.b, (int64_t)tn(it) * TILE, w, lane);
  const uint32_t rl0 = (uint32_t)(uintptr_t)(lds_void_t*)ring;
  auto issue_next = [&](uint32_t st) {
    if (ik == nk) {
      ik = 0;
      it += tstep;
      da = Dma<T, AOp, false>(g.a, (int64_t)tm(it) * TILE, w, lane);
      db = Dma<T, BOp, false>(g.b, (int64_t)tn(it) * TILE, w, lane);
    }
    const int64_t k0 = (int64_t)(ik++) * KST;
    da.issue(st, k0, w, lane);
    db.issue(st + STAGE / 2, k0, w, lane);
  };

  f32x4_t acc[WM][WN];
  f32x4_t colt[WN];  // column terms of this lane's output columns in the current tile
  auto tile_start = [&](int t) {
#pragma unroll
    for (int a = 0; a < WM; ++a)
#pragma unroll
      for (int j = 0; j < WN; ++j) acc[a][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int64_t n0 = (int64_t)tn(t) * TILE;
    if (ctab) {
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int64_t n = n0 + wn * 16 * WN + j * 16 + 4 * fq;
        colt[j] = n + 3 < g.N ? *(const f32x4_t*)(coltab + n) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    } else {
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int64_t n = n0 + wn * 16 * WN + j * 16 + 4 * fq;
        colt[j] = ((g.N & 3) == 0 && n + 3 < g.N) ? g.epi.col4(n) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
      // an explicit wait for these loads (and everything before them), so
      // that the compiler places none of its own in the epilogue inside the
      // stream, where it would also wait for the next tile's ring loads
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
  };
  // Output blocks are written in pairs of 16 x 16 blocks (j0, j1 = j0 + 1):
  // lanes of rows 0-7 keep their j0 values and take the j1 values of the
  // lane 8 rows further (a DPP row rotation by 8), lanes of rows 8-15 the
  // reverse, so that each store covers 8 whole rows of 32 columns (128
  // contiguous bytes each) instead of 16 half rows.
  // one lane's four outputs (m, n..n+3): 16 bytes with the column term
  // (which tile_start fetched exactly for such columns), else one by one
  // through the epilogue, which adds it
  auto store_lane = [&](int64_t m, int64_t n, const f32x4_t& v, const f32x4_t& ct) {
    if (m >= g.M || n >= g.N) return;
    if ((g.N & 3) == 0 && n + 3 < g.N) {
      g.epi.store4(m, n, v + ct);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (n + e >= g.N) break;
        g.epi(m, n + e, v[e]);
      }
    }
  };
  auto epilogue = [&](int t) {
    const int64_t m0 = (int64_t)tm(t) * TILE, n0 = (int64_t)tn(t) * TILE;
    const bool hi = fr >= 8;
#pragma unroll
    for (int a = 0; a < WM; ++a)
#pragma unroll
      for (int jj = 0; jj < WN / 2; ++jj) {
        const int j0 = 2 * jj, j1 = j0 + 1;
        const int64_t mb = m0 + wm * 16 * WM + a * 16;  // first row of the blocks
        const int64_t nb = n0 + wn * 16 * WN + j0 * 16;  // first column of the pair
        if ((g.N & 3) == 0 && nb + 31 < g.N) {
          const f32x4_t v0 = acc[a][j0] + colt[j0], v1 = acc[a][j1] + colt[j1];
          f32x4_t p1;
#pragma unroll
          for (int e = 0; e < 4; ++e) p1[e] = lane_xor8(v1[e]);
          const int r = fr & 7;
          if (mb + r < g.M) g.epi.store4(mb + r, nb + (hi ? 16 : 0) + 4 * fq, hi ? p1 : v0);
          if (mb + 8 + r < g.M) g.epi.store4(mb + 8 + r, nb + (hi ? 0 : 16) + 4 * fq, hi ? v0 : p1);
        } else {
          store_lane(mb + fr, nb + 4 * fq, acc[a][j0], colt[j0]);
          store_lane(mb + fr, nb + 16 + 4 * fq, acc[a][j1], colt[j1]);
        }
      }
  };
  // One stage, as in gemm_lds_kernel with three stages in flight: stage s
  // (slot cur) is complete once at most (stages issued after it) x 4 loads
  // of this wave are outstanding; the bare barrier covers the other waves
  // and frees the slot refilled here.  The slot's offset goes through an
  // empty asm statement, so that the compiler adds it to one set of lane
  // offsets per stage instead of keeping a set of addresses per slot.
  auto stage = [&](int s, int cur) {
    const int after = S - 1 - s;
    if (after >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));
    else if (after == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_s_barrier();
    if (s + NS - 1 < S) issue_next(rl0 + (uint32_t)((cur == 0 ? NS - 1 : cur - 1) * STAGE));
    uint32_t off = (uint32_t)(cur * STAGE);
    asm volatile("" : "+s"(off));
    const char* sa = ring + off;
    const char* sb = sa + STAGE / 2;
    u32x4_t bfv[WN], afv[WM];
#pragma unroll
    for (int j = 0; j < WN; ++j) bfv[j] = frag_krows(sb, wn * 16 * WN + 16 * j + fr, fq);
#pragma unroll
    for (int a = 0; a < WM; ++a) afv[a] = frag_krows(sa, wm * 16 * WM + 16 * a + fr, fq);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int a = 0; a < WM; ++a)
#pragma unroll
      for (int j = 0; j < WN; ++j) acc[a][j] = Mfma<T>::mac(bfv[j], afv[a], acc[a][j]);
    __builtin_amdgcn_sched_barrier(0);
  };

  int ct = tile0;  // tile of the products
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < S) issue_next(rl0 + (uint32_t)(j * STAGE));
  tile_start(ct);
  int s = 0;
  for (int j = 0; j < g.per_wg; ++j) {
    for (int k = 0; k < nk; k += NS, s += NS) {
      stage(s, 0);
      stage(s + 1, 1);
      stage(s + 2, 2);
      stage(s + 3, 3);
    }
    epilogue(ct);
    ct += tstep;
    if (j + 1 < g.per_wg) tile_start(ct);
  }
}

// Split-K sum in a fixed order (split 0, 1, ...), then the epilogue.
template <class Epi>
__global__ void __launch_bounds__(256) splitk_reduce(const float* part, int64_t M, int64_t N, int splits, Epi epi) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * N) return;
  float acc = 0.f;
  for (int sp = 0; sp < splits; ++sp) acc += part[(int64_t)sp * M * N + idx];
  epi(idx / N, idx % N, acc);
}

// Tile and split choice for a product of M x N outputs with K-depth K on
// `cus` compute units: 128 x 128 tiles when they already give one per CU,
// else 64 x 64; then split K (powers of two, >= 4 stages per split) until
// tiles x splits covers the CUs.
struct GemmShape { int tile; int splits; };
static GemmShape choose_shape(int64_t M, int64_t N, int64_t K, int esize, int cus, int max_splits) {
  const int64_t kstage = kRowBytes / esize;
  const int64_t ktiles = (K + kstage - 1) / kstage;
  const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
  const int64_t t64 = ((M + 63) / 64) * ((N + 63) / 64);
  GemmShape gs{t128 >= cus ? 128 : 64, 1};
  const int64_t tiles = gs.tile == 128 ? t128 : t64;
  while (gs.splits < max_splits && tiles * gs.splits < cus && ktiles / (gs.splits * 2) >= 4) gs.splits *= 2;
  return gs;
}

template <typename T, int WM, int WN, class AOp, bool AMN, class BOp, bool BMN, class Epi>
static hipError_t launch_tile(GemmArgs<AOp, BOp, Epi>& g, hipStream_t s) {
  constexpr int BM = 32 * WM, BN = 32 * WN;
  const unsigned gz = (unsigned)g.splits + ((g.zero_words > 0 || g.dsum_out) ? 1u : 0u);
  dim3 grid((unsigned)((g.N + BN - 1) / BN), (unsigned)((g.M + BM - 1) / BM), gz);
  const size_t lds = 2 * (size_t)(BM + BN) * kLdsRow;
  auto fn = gemm_kernel<T, WM, WN, AOp, AMN, BOp, BMN, Epi>;
  hipError_t err = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, s, g);
  return hipGetLastError();
}

// Runs C = A . B through the epilogue; `part` must hold splits*M*N floats
// when the shape splits K.  Optionally clears `zero_bytes` at `zero` in the
// same launch (extra blocks), so that a buffer clear costs no launch.
struct DbDuty { const float* src; void* out; int rows; int64_t cols, H; int dtype; int ijfo; int two; };

template <typename T, class AOp, bool AMN, class BOp, bool BMN, class Epi>
static hipError_t run_gemm(const Plan& p, int64_t M, int64_t N, int64_t K, const AOp& a, const BOp& b,
                           const Epi& e, float* part, void* zero, size_t zero_bytes, hipStream_t s,
                           DbDuty db = DbDuty{nullptr, nullptr, 0, 0, 0, 0, 0, 0}) {
  if (M <= 0 || N <= 0) {
    if (zero_bytes) return launch_fill_zero(zero, zero_bytes, s);
    return hipSuccess;
  }
  const GemmShape gs = choose_shape(M, N, K, (int)sizeof(T), p.cus, part ? p.max_splits : 1);
  constexpr int KSTAGE = kRowBytes / sizeof(T);
  const int64_t ktiles = (K + KSTAGE - 1) / KSTAGE;
  int ktps = (int)((ktiles + gs.splits - 1) / gs.splits);
  if (ktps < 1) ktps = 1;
  GemmArgs<AOp, BOp, Epi> g{M, N, K, ktps, gs.splits, a, b, e, part, (uint32_t*)zero, (int64_t)(zero_bytes / 4),
                            db.src, db.out, db.rows, db.dtype, db.cols, db.H, db.ijfo, db.two, p.nxcd};
  hipError_t err = gs.tile == 128 ? launch_tile<T, 4, 4, AOp, AMN, BOp, BMN, Epi>(g, s)
                                  : launch_tile<T, 2, 2, AOp, AMN, BOp, BMN, Epi>(g, s);
  if (err != hipSuccess || gs.splits == 1) return err;
  const int64_t n = M * N;
  hipLaunchKernelGGL(splitk_reduce<Epi>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, M, N, gs.splits, e);
  return hipGetLastError();
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
// operands of the pipelined path are addressed through buffer descriptors
static bool small_buf(int64_t elems, int esize) { return elems * esize < ((int64_t)1 << 31); }

// Pipelined path (gemm_lds_kernel): K is split in a power of two that
// keeps at least 8 stages per split, chosen by the cost of the launch in
// stage rounds -- waves of work-groups over the CUs times stages per
// work-group, plus the fp32 partials each split writes and the sum reads
// (M x N x 8 bytes; a stage round of all CUs moves about 3.4 MB at the
// HBM rate with 16-bit operands, 6.8 MB with fp32) -- a split taken only
// when it saves a tenth.  (Splitting until the tiles cover the CUs would
// add a second, partial wave of work-groups: 96 tiles of dW on 256 CUs in
// four splits are 1.5 waves, in two splits 0.75.)
// fp32 products take it only for deep K (>= 1024): with a short K the
// 64 x 64 tiles of gemm_kernel cover the CUs without a split-K pass.
template <typename T>
static bool lds_depth_ok(int64_t K) { return sizeof(T) == 2 || K >= 1024; }
template <typename T>
static GemmShape choose_shape_lds(int64_t M, int64_t N, int64_t K, int cus, int max_splits) {
  constexpr int TILE = LdsCfg<T>::kTile;
  const int64_t tiles = ((M + TILE - 1) / TILE) * ((N + TILE - 1) / TILE);
  const int64_t ktiles = K / LdsCfg<T>::kKStage;
  const double round_bytes = sizeof(T) == 2 ? 3.4e6 : 6.8e6;
  auto cost = [&](int s) {
    const int64_t c = cus > 0 ? cus : 1;
    const double rounds = (double)((tiles * s + c - 1) / c), stages = (double)((ktiles + s - 1) / s);
    return rounds * stages + (s > 1 ? (double)s * (double)M * (double)N * 8.0 / round_bytes : 0.0);
  };
  GemmShape gs{TILE, 1};
  for (int s = 2; s <= max_splits && ktiles / s >= 8; s *= 2)
    if (cost(s) < 0.9 * cost(gs.splits)) gs.splits = s;
  return gs;
}

// Tiles per work-group of the persistent form (gemm_lds_multi_kernel) for
// an M x N x K product with both operands k-contiguous, or 1 where it does
// not apply: it needs no split of K, the tiles an exact multiple (>= 2) of
// the CUs, and the stages per tile a multiple of four.
template <typename T>
static int multi_tiles_per_wg(const Plan& p, int64_t M, int64_t N, int64_t K) {
  constexpr int TILE = LdsCfg<T>::kTile;
  const GemmShape gs = choose_shape_lds<T>(M, N, K, p.cus, 1);
  const int64_t tiles = ((M + TILE - 1) / TILE) * ((N + TILE - 1) / TILE);
  const int64_t ktiles = K / LdsCfg<T>::kKStage;
  if (gs.splits != 1 || p.cus <= 0 || p.cus % p.nxcd != 0 || tiles % p.cus != 0 || tiles / p.cus < 2 ||
      ktiles % 4 != 0)
    return 1;
  return (int)(tiles / p.cus);
}

template <typename T, int AMN, int BMN, class AOp, class BOp, class Epi>
static hipError_t run_gemm_lds(const Plan& p, int64_t M, int64_t N, int64_t K, const AOp& a, const BOp& b,
                               const Epi& e, float* part, void* zero, size_t zero_bytes, hipStream_t s,
                               DbDuty db = DbDuty{nullptr, nullptr, 0, 0, 0, 0, 0, 0}) {
  constexpr int TILE = LdsCfg<T>::kTile;
  const GemmShape gs = choose_shape_lds<T>(M, N, K, p.cus, part ? p.max_splits : 1);
  const int64_t ktiles = K / LdsCfg<T>::kKStage;
  int ktps = (int)((ktiles + gs.splits - 1) / gs.splits);
  if (ktps < 1) ktps = 1;
  const int64_t tx = (N + TILE - 1) / TILE, ty = (M + TILE - 1) / TILE;
  GemmArgs<AOp, BOp, Epi> g{M, N, K, ktps, gs.splits, a, b, e, part, (uint32_t*)zero, (int64_t)(zero_bytes / 4),
                            db.src, db.out, db.rows, db.dtype, db.cols, db.H, db.ijfo, db.two, p.nxcd, (int)tx, (int)ty, 1};
  if constexpr (AMN == 0 && BMN == 0) {
    const int per_wg = g.dsum_out ? 1 : multi_tiles_per_wg<T>(p, M, N, K);
    if (per_wg > 1) {
      g.per_wg = per_wg;
      const dim3 grid_m((unsigned)p.cus, 1u, g.zero_words > 0 ? 2u : 1u);
      hipLaunchKernelGGL((gemm_lds_multi_kernel<T, AOp, BOp, Epi>), grid_m, dim3(LdsCfg<T>::kThreads), 0, s, g);
      return hipGetLastError();
    }
  }
  const unsigned gz = (unsigned)gs.splits + ((g.zero_words > 0 || g.dsum_out) ? 1u : 0u);
  dim3 grid((unsigned)tx, (unsigned)ty, gz);
  auto fn = gemm_lds_kernel<T, AMN, BMN, AOp, BOp, Epi>;  // the ring is static LDS
  hipLaunchKernelGGL(fn, grid, dim3(LdsCfg<T>::kThreads), 0, s, g);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || gs.splits == 1) return err;
  const int64_t n = M * N;
  hipLaunchKernelGGL(splitk_reduce<Epi>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, M, N, gs.splits, e);
  return hipGetLastError();
}

// the input projection takes the pipelined path (operands 16-byte aligned)
template <typename T>
static bool inproj_lds_ok(const Plan& p) {
  constexpr int VEC = 16 / sizeof(T);
  return p.I % LdsCfg<T>::kKStage == 0 && lds_depth_ok<T>(p.I) && p.I % VEC == 0 && p.Z % VEC == 0 &&
         p.H % VEC == 0 && p.TB > 0 && small_buf(p.TB * p.I, p.esize) && small_buf(p.G4 * p.Z, p.esize);
}

template <typename T>
static hipError_t inproj_t(const Plan& p, const void* x, const void* W, const void* b, float* P, float* part,
                           void* zero, size_t zero_bytes, hipStream_t s) {
  constexpr int VEC = 16 / sizeof(T);
  KRowsX<T> a{(const T*)x, p.I, p.TB, p.I, aligned16(x) && p.I % VEC == 0};
  KRowsWx<T> bw{(const T*)W, p.H, p.Z, p.G4, p.I, aligned16(W) && p.Z % VEC == 0 && p.H % VEC == 0, p.ijfo};
  EpiP e{P, b, p.H, p.G4, p.dtype, p.ijfo, p.two_bias};
  if (inproj_lds_ok<T>(p) && a.vec_ok && bw.vec_ok)
    return run_gemm_lds<T, 0, 0>(p, p.TB, p.G4, p.I, a, bw, e, part, zero, zero_bytes, s);
  return run_gemm<T, KRowsX<T>, false, KRowsWx<T>, false, EpiP>(p, p.TB, p.G4, p.I, a, bw, e, part, zero, zero_bytes, s);
}

template <typename T, class Epi>
static hipError_t dx_epi(const Plan& p, const void* dG, const void* W, const Epi& e, float* part, void* zero,
                         size_t zero_bytes, hipStream_t s) {
  constexpr int VEC = 16 / sizeof(T);
  KRowsX<T> a{(const T*)dG, p.G4, p.TB, p.G4, aligned16(dG) && p.G4 % VEC == 0};
  MNRowsWx<T> bw{(const T*)W, p.H, p.Z, p.I, p.G4, aligned16(W) && p.Z % VEC == 0 && p.H % VEC == 0, p.ijfo};
  if (p.G4 % LdsCfg<T>::kKStage == 0 && lds_depth_ok<T>(p.G4) && p.I >= VEC && a.vec_ok && bw.vec_ok && p.TB > 0 &&
      small_buf(p.TB * p.G4, p.esize) && small_buf(p.G4 * p.Z, p.esize))
    return run_gemm_lds<T, 0, 1>(p, p.TB, p.I, p.G4, a, bw, e, part, zero, zero_bytes, s);
  return run_gemm<T, KRowsX<T>, false, MNRowsWx<T>, true, Epi>(p, p.TB, p.I, p.G4, a, bw, e, part, zero,
                                                               zero_bytes, s);
}

// dx in the storage type; or its fp32 sums into acc_out; or acc_in plus them
template <typename T>
static hipError_t dx_t(const Plan& p, const void* dG, const void* W, void* dx, float* part, void* zero,
                       size_t zero_bytes, hipStream_t s, float* acc_out, const float* acc_in) {
  if (acc_out) return dx_epi<T>(p, dG, W, EpiStore<float>{acc_out, p.I}, part, zero, zero_bytes, s);
  if (acc_in) return dx_epi<T>(p, dG, W, EpiAdd<T>{(T*)dx, acc_in, p.I}, part, zero, zero_bytes, s);
  return dx_epi<T>(p, dG, W, EpiStore<T>{(T*)dx, p.I}, part, zero, zero_bytes, s);
}

template <typename T>
static hipError_t dw_t(const Plan& p, const void* dG, const void* x, const void* h0, const void* y, void* dW,
                       float* part, void* zero, size_t zero_bytes, const float* DBP, void* db, hipStream_t s) {
  constexpr int VEC = 16 / sizeof(T);
  MNRowsPlain<T> a{(const T*)dG, p.G4, p.G4, p.TB, aligned16(dG) && p.G4 % VEC == 0};
  MNRowsZ<T> bz{(const T*)x, (const T*)h0, (const T*)y, p.B, p.H, p.I, p.Z, p.TB,
                aligned16(x) && aligned16(y) && (h0 == nullptr || aligned16(h0)) && p.H % VEC == 0 && p.I % VEC == 0,
                p.rev != 0};
  EpiDW<T> e{(T*)dW, p.H, p.Z, p.ijfo};
  const DbDuty dd{DBP, db, p.dbp_rows > 0 ? p.dbp_rows : p.nBG, p.G4, p.H, p.dtype, p.ijfo, p.two_bias};
  if (p.TB % LdsCfg<T>::kKStage == 0 && lds_depth_ok<T>(p.TB) && p.Z >= VEC && a.vec_ok && bz.vec_ok &&
      small_buf(p.TB * p.G4, p.esize) && small_buf(p.TB * p.Z, p.esize))
    return run_gemm_lds<T, 1, 1>(p, p.G4, p.Z, p.TB, a, bz, e, part, zero, zero_bytes, s, dd);
  return run_gemm<T, MNRowsPlain<T>, true, MNRowsZ<T>, true, EpiDW<T>>(p, p.G4, p.Z, p.TB, a, bz, e, part, zero,
                                                                       zero_bytes, s, dd);
}

int inproj_tiles_per_wg(const Plan& p) {
  if (p.esize == 2) return inproj_lds_ok<bf16_t>(p) ? multi_tiles_per_wg<bf16_t>(p, p.TB, p.G4, p.I) : 1;
  return inproj_lds_ok<float>(p) ? multi_tiles_per_wg<float>(p, p.TB, p.G4, p.I) : 1;
}

hipError_t launch_gemm_inproj(const Plan& p, const void* x, const void* W, const void* b, float* P, float* part,
                              void* zero, size_t zero_bytes, hipStream_t s) {
  if (p.dtype == 1) return inproj_t<bf16_t>(p, x, W, b, P, part, zero, zero_bytes, s);
  if (p.dtype == 2) return inproj_t<f16_t>(p, x, W, b, P, part, zero, zero_bytes, s);
  return inproj_t<float>(p, x, W, b, P, part, zero, zero_bytes, s);
}
hipError_t launch_gemm_dx(const Plan& p, const void* dG, const void* W, void* dx, float* part, void* zero,
                          size_t zero_bytes, hipStream_t s, float* acc_out, const float* acc_in) {
  if (p.dtype == 1) return dx_t<bf16_t>(p, dG, W, dx, part, zero, zero_bytes, s, acc_out, acc_in);
  if (p.dtype == 2) return dx_t<f16_t>(p, dG, W, dx, part, zero, zero_bytes, s, acc_out, acc_in);
  return dx_t<float>(p, dG, W, dx, part, zero, zero_bytes, s, acc_out, acc_in);
}
hipError_t launch_gemm_dw(const Plan& p, const void* dG, const void* x, const void* h0, const void* y, void* dW,
                          float* part, void* zero, size_t zero_bytes, const float* DBP, void* db, hipStream_t s) {
  if (p.dtype == 1) return dw_t<bf16_t>(p, dG, x, h0, y, dW, part, zero, zero_bytes, DBP, db, s);
  if (p.dtype == 2) return dw_t<f16_t>(p, dG, x, h0, y, dW, part, zero, zero_bytes, DBP, db, s);
  return dw_t<float>(p, dG, x, h0, y, dW, part, zero, zero_bytes, DBP, db, s);
}

// Bytes of fp32 split-K partials the three products need for this plan.
size_t gemm_partial_bytes(const Plan& p, int cus) {
  size_t mx = 0;
  const int64_t shapes[3][3] = {{p.TB, p.G4, p.I}, {p.TB, p.I, p.G4}, {p.G4, p.Z, p.TB}};
  for (const auto& sh : shapes) {
    if (sh[0] <= 0 || sh[1] <= 0) continue;
    GemmShape gs = choose_shape(sh[0], sh[1], sh[2], p.esize, cus, p.max_splits);
    const GemmShape gl = p.esize == 2 ? choose_shape_lds<bf16_t>(sh[0], sh[1], sh[2], cus, p.max_splits)
                                 : choose_shape_lds<float>(sh[0], sh[1], sh[2], cus, p.max_splits);
    if (gl.splits > gs.splits) gs = gl;
    if (gs.splits > 1) {
      const size_t b = (size_t)gs.splits * sh[0] * sh[1] * 4;
      if (b > mx) mx = b;
    }
  }
  return mx;
}

// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) fill_zero_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const int64_t n = (int64_t)(bytes / 4);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t*)p, n);
  return hipGetLastError();
}

// Two directions side by side: row r of `a` and of `b` (rb bytes each) into
// row r of `out` (2*rb bytes), or back (split).  16-byte pieces when the
// rows and pointers allow, else 2-byte ones (every element is 2 or 4 bytes).
template <typename U>
__global__ void __launch_bounds__(256) dirs_kernel(const U* a, const U* b, U* out, int64_t rows, int64_t ru, int split) {
  const int64_t n = rows * ru;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / ru, c = i - r * ru;
    if (split) {
      ((U*)a)[i] = out[r * 2 * ru + c];
      ((U*)b)[i] = out[r * 2 * ru + ru + c];
    } else {
      out[r * 2 * ru + c] = a[i];
      out[r * 2 * ru + ru + c] = b[i];
    }
  }
}
static hipError_t launch_dirs(const void* a, const void* b, void* out, int64_t rows, int64_t rb, int split,
                              hipStream_t s) {
  if (rows <= 0 || rb <= 0) return hipSuccess;
  const bool v16 = rb % 16 == 0 && ((uintptr_t)a | (uintptr_t)b | (uintptr_t)out) % 16 == 0;
  const int64_t ru = v16 ? rb / 16 : rb / 2, n = rows * ru;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (v16)
    hipLaunchKernelGGL(dirs_kernel<u32x4_t>, dim3((unsigned)blocks), dim3(256), 0, s, (const u32x4_t*)a,
                       (const u32x4_t*)b, (u32x4_t*)out, rows, ru, split);
  else
    hipLaunchKernelGGL(dirs_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s, (const uint16_t*)a,
                       (const uint16_t*)b, (uint16_t*)out, rows, ru, split);
  return hipGetLastError();
}
hipError_t launch_join_dirs(const void* y0, const void* y1, void* y, int64_t rows, int64_t row_bytes, hipStream_t s) {
  return launch_dirs(y0, y1, y, rows, row_bytes, 0, s);
}
hipError_t launch_split_dirs(const void* dy, void* dy0, void* dy1, int64_t rows, int64_t row_bytes, hipStream_t s) {
  return launch_dirs(dy0, dy1, const_cast<void*>(dy), rows, row_bytes, 1, s);
}

// dst = src (n elements of esize bytes), or dst = 0 when src is NULL
__global__ void __launch_bounds__(256) copy_state_kernel(const uint8_t* src, uint8_t* dst, int64_t nbytes) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < nbytes) dst[i] = src ? src[i] : (uint8_t)0;
}
hipError_t launch_copy_state(const void* src, void* dst, size_t n, int esize, hipStream_t s) {
  const int64_t nb = (int64_t)n * esize;
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, (const uint8_t*)src,
                     (uint8_t*)dst, nb);
  return hipGetLastError();
}

}  // namespace lstm
