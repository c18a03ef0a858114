// recurrent.hip -- persistent forward and backward recurrences (gfx950).
//
// Forward ("SingleLayerLstmGrad" page, forward table): for t = 0..T-1
//   a_t = P_t + W_h h_{t-1}      (P_t = W_x x_t + b from the input projection)
//   i,f,o = sigmoid, g = tanh;   c_t = f c_{t-1} + i g;   h_t = o tanh(c_t)
// Backward (same page, "反向传播算法" steps 1-6): for t = T-1..0
//   dh = dy_t + dh_carry;  dc = dh o (1 - tanh^2 c_t) + dc_carry
//   do = dh tanh(c_t) o(1-o); dg = dc i (1-g^2); di = dc g i(1-i);
//   df = dc c_{t-1} f(1-f);  dc_carry = dc f;  dh_carry = W_h^T dG_t
// with dh_carry/dc_carry starting from dhT/dcT, and dh0/dc0 the carries
// left after t = 0.
//
// One launch per direction of time; the grid (nBG x nJG work-groups, one
// per CU, co-resident by cooperative launch) runs every step.  Work-group
// (bg, jg) owns batch rows [bg*NB, +NB) and hidden units [jg*NJ, +NJ); it
// keeps the 4*NJ rows of W_h that belong to its units (gates i,f,g,o of each
// unit) in VGPRs as MFMA fragments for the whole launch.  Batch groups never
// talk to each other: rows of the batch are independent in both passes.
//
// Rows are interleaved: MFMA row 4u + g is gate g of unit u, so one lane
// holds the four gates of one (unit, batch) pair after each product and the
// cell update needs no data movement.
//
// Exchange per step inside a batch group, through tagged 8-byte words
// (value + step tag, relaxed agent-scope atomics; see device_common.hpp):
//   forward:  h_t of the group's rows (each work-group writes its units);
//   backward: each work-group writes the fp32 partial product
//             W_h[rows of its units]^T dG_t for all H columns, and every
//             work-group sums, in a fixed order, the partials of its own
//             units from all work-groups of the group.
// No other grid-wide synchronisation is used.
#include "device_common.hpp"
#include "internal.hpp"

namespace lstm {

constexpr int kRecThreads = 256;
constexpr int kMaxKb = 32;   // max k-blocks of W_h fragments per wave (128 VGPRs)
constexpr int kChunk = 16;   // exchange words in flight per thread

struct FwdArgs {
  const float* P;   // [TB][4H] fp32, interleaved gates, bias included
  const void* W;    // [4H][H+I]
  const void* h0;   // [B][H] or null
  const void* c0;   // [B][H] or null
  void* y;          // [T][B][H]
  void* hT;         // [B][H]
  void* cT;         // [B][H]
  void* Gs;         // [TB][4H] activated gates, interleaved
  float* Cs;        // [TB][H] cell states
  uint64_t* HX;     // [2][Bp][HW] exchange words
  uint32_t* err;
  int T, B, H, Z, NB, NJ, nJG, Hp, Bp, HW;
};

struct BwdArgs {
  const void* W;
  const void* c0;
  const void* dy;   // [T][B][H]
  const void* dhT;  // [B][H] or null
  const void* dcT;  // [B][H] or null
  const void* Gs;
  const float* Cs;
  void* dG;         // [TB][4H] gate deltas, interleaved
  uint64_t* PX;     // [2][nJG][Hp][Bp] exchange words (fp32 partials)
  void* dh0;
  void* dc0;
  uint32_t* err;
  int T, B, H, Z, NB, NJ, nJG, Hp, Bp;
};

// Bounded wait for a tagged word.  Returns the word (whatever it holds if
// the wait timed out; then the error word is set and `dead` makes every
// later wait of this thread return at once).
__device__ __forceinline__ uint64_t wait_word(const uint64_t* p, uint64_t w, uint32_t tag, uint32_t* err,
                                              bool& dead) {
  if (xtag(w) == tag || dead) return w;
  const uint64_t t0 = now_ticks();
  int n = 0;
  while (true) {
    w = xload(p);
    if (xtag(w) == tag) return w;
    if (++n == 64) {
      n = 0;
      if (now_ticks() - t0 > kWaitTicks || __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        atomicOr(err, kErrTimeout);
        dead = true;
        return w;
      }
    }
  }
}

template <typename T>
__device__ __forceinline__ float ldf(const void* p, int64_t i) {
  return Elem<T>::to_f(((const T*)p)[i]);
}

// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(kRecThreads, 1) fwd_rec_kernel(FwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int E = sizeof(T);
  constexpr int KB = Mfma<T>::kBlock;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int fr = lane & 15, fq = lane >> 4;
  const int bg = blockIdx.x / a.nJG, jg = blockIdx.x % a.nJG;
  const int b0 = bg * a.NB, j0 = jg * a.NJ;
  const int MT = a.NJ / 4, NBT = a.NB / 16;  // M-tiles (16 gate rows), N-tiles (16 batch rows)
  const int KS = 4 / MT;                     // waves splitting k per M-tile
  const int mt = w / KS, wk = w % KS;        // this wave's M-tile and k part
  const int nkb = a.Hp / KB, nkbw = nkb / KS, kb0 = wk * nkbw;
  const int strideH = a.Hp * E + 16;         // LDS row of h_{t-1}
  char* Hl = smem;                           // [NB][strideH]
  float* red = (float*)(smem + a.NB * strideH);  // [4 waves][NBT][64][4]
  const int64_t G4 = 4 * (int64_t)a.H;
  bool dead = false;

  // --- resident W_h fragments: rows 16*mt + fr (gate fr&3 of unit 4*mt + fr/4)
  u32x4_t wreg[kMaxKb];
  {
    const int u = j0 + 4 * mt + (fr >> 2), g = fr & 3;
    const T* wrow = (const T*)a.W + ((int64_t)g * a.H + u) * a.Z;
#pragma unroll
    for (int i = 0; i < kMaxKb; ++i) {
      wreg[i] = u32x4_t{0, 0, 0, 0};
      if (i < nkbw) {
        T tmp[16 / E];
        const int k = (kb0 + i) * KB + fq * (16 / E);
#pragma unroll
        for (int e = 0; e < 16 / E; ++e) tmp[e] = (u < a.H && k + e < a.H) ? wrow[k + e] : T(0);
        wreg[i] = __builtin_bit_cast(u32x4_t, tmp);
      }
    }
  }
  // --- zero the padding of h_{t-1} in LDS once (k >= H, rows past B)
  for (int idx = tid; idx < a.NB * a.Hp; idx += kRecThreads) {
    const int bl = idx / a.Hp, k = idx % a.Hp;
    if (k >= a.H || b0 + bl >= a.B) *(T*)(Hl + bl * strideH + k * E) = T(0);
  }
  // --- cell state of this lane's elements (wk == 0 waves own the elementwise)
  float cst[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    cst[nt] = 0.f;
    const int u = j0 + 4 * mt + fq, b = b0 + 16 * nt + fr;
    if (nt < NBT && a.c0 && u < a.H && b < a.B) cst[nt] = ldf<T>(a.c0, (int64_t)b * a.H + u);
  }
  const int NBv = (a.B - b0) < a.NB ? (a.B - b0) : a.NB;  // valid rows of this group
  const int vpw = (E == 2) ? 2 : 1;                      // values per exchange word

  for (int t = 0; t < a.T; ++t) {
    // prefetch the input projection of this lane's elements
    f32x4_t pf[4];
    if (wk == 0) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        pf[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int u = j0 + 4 * mt + fq, b = b0 + 16 * nt + fr;
        if (nt < NBT && u < a.H && b < a.B)
          pf[nt] = *(const f32x4_t*)(a.P + ((int64_t)t * a.B + b) * G4 + 4 * (int64_t)u);
      }
    }
    __syncthreads();  // previous step's readers of Hl are done
    // h_{t-1} -> LDS
    if (t == 0) {
      for (int idx = tid; idx < NBv * a.H; idx += kRecThreads) {
        const int bl = idx / a.H, k = idx % a.H;
        const T v = a.h0 ? ((const T*)a.h0)[(int64_t)(b0 + bl) * a.H + k] : T(0);
        *(T*)(Hl + bl * strideH + k * E) = v;
      }
    } else {
      const uint64_t* src = a.HX + (int64_t)((t - 1) & 1) * a.Bp * a.HW;
      const int HWv = (a.H + vpw - 1) / vpw;
      const int total = NBv * HWv;
      const uint32_t tag = (uint32_t)t;
      for (int base = 0; base < total; base += kRecThreads * kChunk) {
        uint64_t wv[kChunk];
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          const int idx = base + c * kRecThreads + tid;
          if (idx < total) wv[c] = xload(src + (int64_t)(b0 + idx / HWv) * a.HW + idx % HWv);
        }
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          const int idx = base + c * kRecThreads + tid;
          if (idx < total) {
            const int bl = idx / HWv, kw = idx % HWv;
            const uint64_t* p = src + (int64_t)(b0 + bl) * a.HW + kw;
            const uint64_t v = wait_word(p, wv[c], tag, a.err, dead);
            if constexpr (E == 2) {
              *(uint32_t*)(Hl + bl * strideH + kw * 4) = (uint32_t)v;  // two bf16 values
            } else {
              *(float*)(Hl + bl * strideH + kw * 4) = xval(v);
            }
          }
        }
      }
    }
    __syncthreads();

    // MFMA: acc[nt] = W_h[rows of M-tile mt, k part] . h_{t-1}[tile nt]^T
    f32x4_t acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kMaxKb; ++i) {
      if (i < nkbw) {
        const int kb = kb0 + i;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          if (nt < NBT) {
            const u32x4_t hb = *(const u32x4_t*)(Hl + (16 * nt + fr) * strideH + kb * 64 + fq * 16);
            acc[nt] = Mfma<T>::mac(wreg[i], hb, acc[nt]);
          }
        }
      }
    }
    if (KS > 1) {
      if (wk != 0) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          if (nt < NBT) *(f32x4_t*)(red + ((w * 4 + nt) * 64 + lane) * 4) = acc[nt];
      }
      __syncthreads();
      if (wk == 0) {
        for (int k2 = 1; k2 < KS; ++k2) {
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            if (nt < NBT) {
              const f32x4_t o = *(const f32x4_t*)(red + (((w + k2) * 4 + nt) * 64 + lane) * 4);
              acc[nt] += o;
            }
        }
      }
    }

    // elementwise: gates, cell, hidden; outputs and the exchange word
    if (wk == 0) {
      const int u = j0 + 4 * mt + fq;
      uint64_t* dst = a.HX + (int64_t)(t & 1) * a.Bp * a.HW;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if (nt < NBT) {
          const int b = b0 + 16 * nt + fr;
          const bool valid = u < a.H && b < a.B;
          const f32x4_t z = acc[nt] + pf[nt];
          const float ig = sigmoidf(z[0]), fg = sigmoidf(z[1]), gg = tanh_f(z[2]), og = sigmoidf(z[3]);
          const float c = fg * cst[nt] + ig * gg;
          const float h = og * tanh_f(c);
          cst[nt] = c;
          const T hq = Elem<T>::from_f(h);
          const float hv = Elem<T>::to_f(hq);
          const int64_t o = (int64_t)t * a.B + b;
          if (valid) {
            ((T*)a.y)[o * a.H + u] = hq;
            T gq[4] = {Elem<T>::from_f(ig), Elem<T>::from_f(fg), Elem<T>::from_f(gg), Elem<T>::from_f(og)};
            if constexpr (E == 4)
              *(f32x4_t*)((T*)a.Gs + o * G4 + 4 * (int64_t)u) = __builtin_bit_cast(f32x4_t, gq);
            else
              *(uint64_t*)((T*)a.Gs + o * G4 + 4 * (int64_t)u) = __builtin_bit_cast(uint64_t, gq);
            a.Cs[o * a.H + u] = c;
            if (t == a.T - 1) {
              ((T*)a.hT)[(int64_t)b * a.H + u] = hq;
              ((T*)a.cT)[(int64_t)b * a.H + u] = Elem<T>::from_f(c);
            }
          }
          if constexpr (E == 2) {
            // pack units u (even lane group) and u+1 (next lane group) into one word
            const uint32_t mine = (uint32_t)__builtin_bit_cast(uint16_t, hq);
            const uint32_t next = (uint32_t)__shfl_down((int)mine, 16, 64);
            if ((fq & 1) == 0 && valid) {
              const uint32_t both = mine | ((u + 1 < a.H) ? (next << 16) : 0u);
              __hip_atomic_store(dst + (int64_t)b * a.HW + u / 2, ((uint64_t)(t + 1) << 32) | both,
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          } else {
            if (valid) xstore(dst + (int64_t)b * a.HW + u, hv, (uint32_t)(t + 1));
          }
        }
      }
    }
  }
  // T == 0 is handled on the host
}

// ---------------------------------------------------------------------------
template <typename T, int NKBR>
__global__ void __launch_bounds__(kRecThreads, 1) bwd_rec_kernel(BwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int E = sizeof(T);
  constexpr int KB = Mfma<T>::kBlock;
  constexpr int MAXMT = kMaxKb / NKBR;  // column tiles of W_h^T per wave held in VGPRs
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int fr = lane & 15, fq = lane >> 4;
  const int bg = blockIdx.x / a.nJG, jg = blockIdx.x % a.nJG;
  const int b0 = bg * a.NB, j0 = jg * a.NJ;
  const int R = 4 * a.NJ;                 // gate rows of this group's units
  const int NBT = a.NB / 16;
  const int nMT = a.Hp / 16;              // 16-column tiles of the partial product
  const int mtw = (nMT + 3) / 4;          // per wave (round-robin: tile = w + 4*i)
  const int strideD = R * E + 16;
  char* Dl = smem;                        // [NB][strideD] gate deltas (B operand)
  const int64_t G4 = 4 * (int64_t)a.H;
  bool dead = false;

  // --- resident fragments of W_h^T: A[m = column k][kslot = row r]
  u32x4_t wreg[kMaxKb];
#pragma unroll
  for (int i = 0; i < MAXMT; ++i) {
#pragma unroll
    for (int kb = 0; kb < NKBR; ++kb) {
      u32x4_t v = {0, 0, 0, 0};
      const int mtile = w + 4 * i;
      if (i < mtw && mtile < nMT) {
        const int k = 16 * mtile + fr;  // column of W_h
        T tmp[16 / E];
#pragma unroll
        for (int e = 0; e < 16 / E; ++e) {
          const int r = kb * KB + fq * (16 / E) + e;  // interleaved row: unit r/4, gate r%4
          const int u = j0 + (r >> 2), g = r & 3;
          tmp[e] = (k < a.H && u < a.H && r < R) ? ((const T*)a.W)[((int64_t)g * a.H + u) * a.Z + k] : T(0);
        }
        v = __builtin_bit_cast(u32x4_t, tmp);
      }
      wreg[i * NKBR + kb] = v;
    }
  }

  // --- elementwise ownership: elements e = tid + 256*s, batch fastest
  const int nel = a.NB * a.NJ;
  float dcc[4], dhc[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int e = tid + kRecThreads * s;
    const int bl = e % a.NB, jj = e / a.NB;
    const int b = b0 + bl, u = j0 + jj;
    const bool valid = e < nel && b < a.B && u < a.H;
    dcc[s] = (valid && a.dcT) ? ldf<T>(a.dcT, (int64_t)b * a.H + u) : 0.f;
    dhc[s] = (valid && a.dhT) ? ldf<T>(a.dhT, (int64_t)b * a.H + u) : 0.f;
  }

  for (int t = a.T - 1; t >= -1; --t) {
    // 1. gather dh_carry: sum over work-groups of the partials produced at step t+1
    if (t < a.T - 1) {
      const uint64_t* src = a.PX + (int64_t)((t + 1) & 1) * a.nJG * a.Hp * a.Bp;
      const uint32_t tag = (uint32_t)(t + 2);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int e = tid + kRecThreads * s;
        const int bl = e % a.NB, jj = e / a.NB;
        const int b = b0 + bl, u = j0 + jj;
        if (e < nel && b < a.B && u < a.H) {
          float sum = 0.f;
          for (int base = 0; base < a.nJG; base += kChunk) {
            uint64_t wv[kChunk];
#pragma unroll
            for (int c = 0; c < kChunk; ++c)
              if (base + c < a.nJG) wv[c] = xload(src + ((int64_t)(base + c) * a.Hp + u) * a.Bp + b);
#pragma unroll
            for (int c = 0; c < kChunk; ++c)
              if (base + c < a.nJG) {
                const uint64_t* p = src + ((int64_t)(base + c) * a.Hp + u) * a.Bp + b;
                sum += xval(wait_word(p, wv[c], tag, a.err, dead));
              }
          }
          dhc[s] = sum;
        }
      }
    }
    if (t < 0) break;

    // 2. gate deltas of this step
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int e = tid + kRecThreads * s;
      if (e < nel) {
        const int bl = e % a.NB, jj = e / a.NB;
        const int b = b0 + bl, u = j0 + jj;
        T dq[4] = {T(0), T(0), T(0), T(0)};
        if (b < a.B && u < a.H) {
          const int64_t o = (int64_t)t * a.B + b;
          float gi, gf, gg, go;
          if constexpr (E == 4) {
            const f32x4_t gv = *(const f32x4_t*)((const T*)a.Gs + o * G4 + 4 * (int64_t)u);
            gi = gv[0]; gf = gv[1]; gg = gv[2]; go = gv[3];
          } else {
            const uint64_t raw = *(const uint64_t*)((const T*)a.Gs + o * G4 + 4 * (int64_t)u);
            gi = bf2f((bf16_t)raw); gf = bf2f((bf16_t)(raw >> 16)); gg = bf2f((bf16_t)(raw >> 32)); go = bf2f((bf16_t)(raw >> 48));
          }
          const float c = a.Cs[o * a.H + u];
          const float cprev = t > 0 ? a.Cs[(o - a.B) * a.H + u] : (a.c0 ? ldf<T>(a.c0, (int64_t)b * a.H + u) : 0.f);
          const float tc = tanh_f(c);
          const float dh = ldf<T>(a.dy, o * a.H + u) + dhc[s];
          const float dc = dh * go * (1.f - tc * tc) + dcc[s];
          const float d_o = dh * tc * go * (1.f - go);
          const float d_g = dc * gi * (1.f - gg * gg);
          const float d_i = dc * gg * gi * (1.f - gi);
          const float d_f = dc * cprev * gf * (1.f - gf);
          dcc[s] = dc * gf;
          dq[0] = Elem<T>::from_f(d_i); dq[1] = Elem<T>::from_f(d_f);
          dq[2] = Elem<T>::from_f(d_g); dq[3] = Elem<T>::from_f(d_o);
          if constexpr (E == 4)
            *(f32x4_t*)((T*)a.dG + o * G4 + 4 * (int64_t)u) = __builtin_bit_cast(f32x4_t, dq);
          else
            *(uint64_t*)((T*)a.dG + o * G4 + 4 * (int64_t)u) = __builtin_bit_cast(uint64_t, dq);
        }
        if constexpr (E == 4)
          *(f32x4_t*)(Dl + bl * strideD + jj * 16) = __builtin_bit_cast(f32x4_t, dq);
        else
          *(uint64_t*)(Dl + bl * strideD + jj * 8) = __builtin_bit_cast(uint64_t, dq);
      }
    }
    __syncthreads();

    // 3. partial[k][b] = sum_{r in my rows} W_h[r][k] dG[b][r], all k < H
    uint64_t* dst = a.PX + ((int64_t)(t & 1) * a.nJG + jg) * a.Hp * a.Bp;
    for (int nt = 0; nt < NBT; ++nt) {
      u32x4_t breg[NKBR];
#pragma unroll
      for (int kb = 0; kb < NKBR; ++kb)
        breg[kb] = *(const u32x4_t*)(Dl + (16 * nt + fr) * strideD + kb * 64 + fq * 16);
      const int b = b0 + 16 * nt + fr;
#pragma unroll
      for (int i = 0; i < MAXMT; ++i) {
        const int mtile = w + 4 * i;
        if (i < mtw && mtile < nMT) {
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < NKBR; ++kb) acc = Mfma<T>::mac(wreg[i * NKBR + kb], breg[kb], acc);
          if (b < a.B) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int k = 16 * mtile + 4 * fq + e;
              if (k < a.H) xstore(dst + (int64_t)k * a.Bp + b, acc[e], (uint32_t)(t + 1));
            }
          }
        }
      }
    }
    __syncthreads();  // Dl is rewritten next step
  }

  // dh0 / dc0
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int e = tid + kRecThreads * s;
    const int bl = e % a.NB, jj = e / a.NB;
    const int b = b0 + bl, u = j0 + jj;
    if (e < nel && b < a.B && u < a.H) {
      ((T*)a.dh0)[(int64_t)b * a.H + u] = Elem<T>::from_f(dhc[s]);
      ((T*)a.dc0)[(int64_t)b * a.H + u] = Elem<T>::from_f(dcc[s]);
    }
  }
}

// ---------------------------------------------------------------------------
template <typename K>
static hipError_t coop_launch(K kernel, int grid, size_t lds, void* arg, hipStream_t s) {
  hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  void* args[] = {arg};
  return hipLaunchCooperativeKernel((const void*)kernel, dim3(grid), dim3(kRecThreads), args, (unsigned)lds, s);
}

hipError_t launch_fwd_recurrent(const Plan& p, const float* P, const void* W, const void* h0, const void* c0,
                                void* y, void* hT, void* cT, void* Gs, float* Cs, uint64_t* HX, uint32_t* err,
                                hipStream_t s) {
  FwdArgs a{P, W, h0, c0, y, hT, cT, Gs, Cs, HX, err, (int)p.T, (int)p.B, (int)p.H, (int)p.Z, p.NB, p.NJ, p.nJG,
            p.Hp, p.Bp, p.dtype ? (p.Hp / 2) : p.Hp};
  if (p.dtype) return coop_launch(fwd_rec_kernel<bf16_t>, p.grid, p.lds_fwd, &a, s);
  return coop_launch(fwd_rec_kernel<float>, p.grid, p.lds_fwd, &a, s);
}

hipError_t launch_bwd_recurrent(const Plan& p, const void* W, const void* c0, const void* dy, const void* dhT,
                                const void* dcT, const void* Gs, const float* Cs, void* dG, uint64_t* PX, void* dh0,
                                void* dc0, uint32_t* err, hipStream_t s) {
  BwdArgs a{W, c0, dy, dhT, dcT, Gs, Cs, dG, PX, dh0, dc0, err, (int)p.T, (int)p.B, (int)p.H, (int)p.Z,
            p.NB, p.NJ, p.nJG, p.Hp, p.Bp};
  const int nkbr = 4 * p.NJ * p.esize / 64;
  if (p.dtype) {
    if (nkbr == 1) return coop_launch(bwd_rec_kernel<bf16_t, 1>, p.grid, p.lds_bwd, &a, s);
    if (nkbr == 2) return coop_launch(bwd_rec_kernel<bf16_t, 2>, p.grid, p.lds_bwd, &a, s);
  } else {
    if (nkbr == 2) return coop_launch(bwd_rec_kernel<float, 2>, p.grid, p.lds_bwd, &a, s);
    if (nkbr == 4) return coop_launch(bwd_rec_kernel<float, 4>, p.grid, p.lds_bwd, &a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace lstm
