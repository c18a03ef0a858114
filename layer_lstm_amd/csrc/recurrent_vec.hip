// recurrent_vec.hip -- forward recurrence for fp32 storage with batch groups
// of at most 4 rows, the product on the vector ALUs (gfx950).
//
// Same step as the MFMA kernel ("SingleLayerLstmGrad" page, forward table:
// a_t = P_t + W_h h_{t-1}; i,f,o = sigmoid, g = tanh; c_t = f c_{t-1} + i g;
// h_t = o tanh(c_t)), but a 16x16 MFMA tile would leave 12 of its 16 batch
// columns empty for 4 rows.  Here:
//   lane c (0..31) of half-wave h of wave w owns local unit 2w + h (+ 8q for
//   q < U2 when NJ = 16): the four gate rows of the unit over the k-chunk c
//   of L = max(4, Hp/32) columns, kept in VGPRs for the whole launch;
//   h_{t-1} of the 4 rows sits in LDS as [row][chunk][L + 4] (the pad puts
//   neighbouring chunks on different banks);
//   each lane forms the 16 (gate, row) dot-product pieces of its chunk with
//   fp32 FMAs -- per FMA one LDS value feeds four gates, which keeps the
//   LDS reads (not the FMAs) from bounding the step;
//   the 32 chunks are summed by a reduce-scatter across the half-wave (xor
//   16 by ds_swizzle; xor 8, 4, 2, 1 by DPP), after which lane c holds the
//   full sum of gate 2*c[2] + c[1] for batch row 2*c[4] + c[3];
//   lane c = 8b (b < 4) gathers the four gates of batch row b by DPP and
//   does the cell update of that (unit, row) element.
// The exchange (tagged words, XCD-local or device-wide) is the same as in
// recurrent.hip.
#include "recurrent_common.hpp"

namespace lstm {

// gfx9 DPP controls
constexpr int kQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadBcast2 = 0xAA;  // quad_perm [2,2,2,2]
constexpr int kRowShl4 = 0x104, kRowShl8 = 0x108, kRowShr4 = 0x114, kRowShr8 = 0x118;

// v from another lane by a DPP move; lanes outside bank_mask keep `old`.
template <int CTRL, int BANKS = 0xf>
__device__ __forceinline__ float dpp_f32(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                                               CTRL, 0xf, BANKS, false));
}
// v of lane l ^ 8 (inside a 16-lane row): lanes 8..15 take from l - 8,
// lanes 0..7 from l + 8.
__device__ __forceinline__ float xor8_f32(float v) { return dpp_f32<kRowShl8, 0x3>(dpp_f32<kRowShr8, 0xC>(0.f, v), v); }
// v of lane l ^ 4: banks 1, 3 (lane bit 2 set) take from l - 4, banks 0, 2 from l + 4.
__device__ __forceinline__ float xor4_f32(float v) { return dpp_f32<kRowShl4, 0x5>(dpp_f32<kRowShr4, 0xA>(0.f, v), v); }
// v of lane l ^ 16 (within each 32-lane half), ds_swizzle bit mode.
__device__ __forceinline__ float xor16_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

template <int L, int U2, int C>
__global__ void __launch_bounds__(kRecThreads, 1) fwd_vec_kernel(FwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) float hl[];
  constexpr int CS = L + 4;    // chunk stride (floats)
  constexpr int RS = 32 * CS;  // row stride
  constexpr int LG_L = L == 4 ? 2 : L == 8 ? 3 : L == 16 ? 4 : 5;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int bg, jg;
  take_role(a.nBG, a.nJG, a.nxcd, a.local, bg, jg);
  const bool local = a.local != 0;
  const int b0 = bg * a.NB, j0 = jg * a.NJ;  // NB == 4
  const int c = lane & 31, ulb = 2 * w + (lane >> 5);
  const int bit4 = (c >> 4) & 1, bit3 = (c >> 3) & 1, bit2 = (c >> 2) & 1, bit1 = (c >> 1) & 1;
  const int64_t G4 = 4 * (int64_t)a.H;
  bool dead = false;

  // resident W_h: gates 0..3 of units j0 + ulb + 8q, columns of chunk c
  float wr[U2][4][L];
#pragma unroll
  for (int q = 0; q < U2; ++q) {
    const int ur = j0 + ulb + 8 * q;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float* wrow = (const float*)a.W + ((int64_t)g * a.H + ur) * a.Z;
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const int k = c * L + i;
        wr[q][g][i] = (ur < a.H && k < a.H) ? wrow[k] : 0.f;
      }
    }
  }
  const int NBv = (a.B - b0) < 4 ? (a.B - b0) : 4;
  for (int idx = tid; idx < 4 * RS; idx += kRecThreads) hl[idx] = 0.f;

  // elementwise lanes: c = 8b -> batch row b
  const int bme_l = c >> 3;
  const bool ew = (c & 7) == 0 && bme_l < NBv;
  const int bme = b0 + bme_l;
  float cst[U2];
  f32x4_t pf[U2];
#pragma unroll
  for (int q = 0; q < U2; ++q) {
    const int u = j0 + ulb + 8 * q;
    cst[q] = (ew && a.c0 && u < a.H) ? ((const float*)a.c0)[(int64_t)bme * a.H + u] : 0.f;
  }
  auto load_p = [&](int tt) {
#pragma unroll
    for (int q = 0; q < U2; ++q) {
      const int u = j0 + ulb + 8 * q;
      pf[q] = (ew && tt < a.T && u < a.H) ? *(const f32x4_t*)(a.P + ((int64_t)tt * a.B + bme) * G4 + 4 * (int64_t)u)
                                          : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  load_p(0);

  const int lgHW = 31 - __builtin_clz(a.HW);  // HW = Hp words per row
  const int total = NBv << lgHW;
  const uint32_t doff = (uint32_t)(tid % total);

  for (int t = 0; t < a.T; ++t) {
    stamp(a.stamps, a.T, t, 0);
    const uint64_t* src = a.HX + ((int64_t)((t - 1) & 1) * a.Bp + b0) * a.HW;
    uint32_t off[C];
    uint32_t live = 0;
    uint64_t wv[C];
    if (t > 0) {
      live = plan_h_round<C>(off, 0, tid, total, a.HW - 1, a.H, doff);
      issue_tagged<C>(wv, src, off);
    }
    __syncthreads();  // the previous step's readers of hl are done
    if (t == 0) {
      wait_vmem();
      for (int idx = tid; idx < NBv * a.H; idx += kRecThreads) {
        const int bl = idx / a.H, k = idx % a.H;
        hl[bl * RS + (k >> LG_L) * CS + (k & (L - 1))] = a.h0 ? ((const float*)a.h0)[(int64_t)(b0 + bl) * a.H + k] : 0.f;
      }
    } else {
      for (int base = 0;;) {
        complete_tagged<C>(wv, src, off, live, (uint32_t)t, a.err, dead);
#pragma unroll
        for (int cc = 0; cc < C; ++cc) {
          if ((live >> cc) & 1u) {
            const int bl = off[cc] >> lgHW, k = off[cc] & (a.HW - 1);
            hl[bl * RS + (k >> LG_L) * CS + (k & (L - 1))] = xval(wv[cc]);
          }
        }
        base += kRecThreads * C;
        if (base >= total) break;
        live = plan_h_round<C>(off, base, tid, total, a.HW - 1, a.H, doff);
        issue_tagged<C>(wv, src, off);
      }
    }
    // Everything this wave issued before (last step's stores, the input
    // prefetch) has completed by now; saying so keeps the compiler from
    // waiting for stores before it reuses their registers below.
    wait_vmem();
    stamp(a.stamps, a.T, t, 1);
    __syncthreads();
    stamp(a.stamps, a.T, t, 2);

    // dot-product pieces of chunk c: acc[q][g][b]
    float acc[U2][4][4];
#pragma unroll
    for (int q = 0; q < U2; ++q)
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[q][g][0] = acc[q][g][1] = acc[q][g][2] = acc[q][g][3] = 0.f;
    const float* hb = hl + c * CS;
#pragma unroll
    for (int i4 = 0; i4 < L / 4; ++i4) {
      f32x4_t hv[4];
#pragma unroll
      for (int bl = 0; bl < 4; ++bl) hv[bl] = *(const f32x4_t*)(hb + bl * RS + 4 * i4);
#pragma unroll
      for (int q = 0; q < U2; ++q)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int bl = 0; bl < 4; ++bl)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc[q][g][bl] = fmaf(wr[q][g][4 * i4 + kk], hv[bl][kk], acc[q][g][bl]);
    }
    stamp(a.stamps, a.T, t, 3);

    // reduce-scatter over the 32 chunk lanes; then gather the four gates
    f32x4_t z[U2];
#pragma unroll
    for (int q = 0; q < U2; ++q) {
      // bit 4: keep rows 2*bit4 + {0,1}
      float k8[4][2];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const float keep = bit4 ? acc[q][g][2 + bb] : acc[q][g][bb];
          const float send = bit4 ? acc[q][g][bb] : acc[q][g][2 + bb];
          k8[g][bb] = keep + xor16_f32(send);
        }
      // bit 3: keep row 2*bit4 + bit3
      float k4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float keep = bit3 ? k8[g][1] : k8[g][0];
        const float send = bit3 ? k8[g][0] : k8[g][1];
        k4[g] = keep + xor8_f32(send);
      }
      // bit 2: keep gates 2*bit2 + {0,1}
      float k2[2];
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const float keep = bit2 ? k4[2 + gg] : k4[gg];
        const float send = bit2 ? k4[gg] : k4[2 + gg];
        k2[gg] = keep + xor4_f32(send);
      }
      // bit 1: keep gate 2*bit2 + bit1; bit 0: both lanes of the pair sum
      const float keep = bit1 ? k2[1] : k2[0];
      const float send = bit1 ? k2[0] : k2[1];
      float v = keep + dpp_f32<kQuadSwap2>(0.f, send);
      v += dpp_f32<kQuadSwap1>(0.f, v);
      // lane 8b + 2*bit2 + bit1 now holds gate 2*bit2 + bit1 of row b
      const float g1 = dpp_f32<kQuadBcast2>(0.f, v);  // from lane + 2
      z[q][0] = v;
      z[q][1] = g1;
      z[q][2] = dpp_f32<kRowShl4>(0.f, v);   // from lane + 4
      z[q][3] = dpp_f32<kRowShl4>(0.f, g1);  // from lane + 6
    }
    stamp(a.stamps, a.T, t, 4);

    if (ew) {
      uint64_t* dst = a.HX + (int64_t)(t & 1) * a.Bp * a.HW;
#pragma unroll
      for (int q = 0; q < U2; ++q) {
        const int u = j0 + ulb + 8 * q;
        if (u < a.H) {
          const f32x4_t zz = z[q] + pf[q];
          const float ig = sigmoidf(zz[0]), fg = sigmoidf(zz[1]), gg = tanh_f(zz[2]), og = sigmoidf(zz[3]);
          const float cn = fg * cst[q] + ig * gg;
          const float h = og * tanh_f(cn);
          cst[q] = cn;
          xstore(dst + (int64_t)bme * a.HW + u, h, (uint32_t)(t + 1), local);
          const int64_t o = (int64_t)t * a.B + bme;
          ((float*)a.y)[o * a.H + u] = h;
          *(f32x4_t*)((float*)a.Gs + o * G4 + 4 * (int64_t)u) = f32x4_t{ig, fg, gg, og};
          a.Cs[o * a.H + u] = cn;
          if (t == a.T - 1) {
            ((float*)a.hT)[(int64_t)bme * a.H + u] = h;
            ((float*)a.cT)[(int64_t)bme * a.H + u] = cn;
          }
        }
      }
    }
    load_p(t + 1);
    stamp(a.stamps, a.T, t, 5);
  }
}

// Dispatch: L = max(4, Hp/32) columns per chunk, U2 = NJ/8 units per
// half-wave; the resident slice 4*U2*L floats per lane is kept at most 64
// (larger slices spill with the fully unrolled product).
static int vec_chunk(const Plan& p) { return p.Hp / 32 < 4 ? 4 : p.Hp / 32; }

bool fwd_vec_ok(const Plan& p) {
  if (p.dtype != 0 || p.NB != 4) return false;
  const int L = vec_chunk(p), u2 = p.NJ / 8;
  return L <= 16 && (u2 == 1 || u2 == 2) && 4 * u2 * L <= 64;
}

template <int U2, int C>
static hipError_t fwd_vec_l(const Plan& p, FwdArgs& a, hipStream_t s) {
  const int L = vec_chunk(p);
  const size_t lds = (size_t)4 * 32 * (L + 4) * sizeof(float);
  switch (L) {
    case 4: return coop_launch(fwd_vec_kernel<4, U2, C>, p.grid, lds, &a, s);
    case 8: return coop_launch(fwd_vec_kernel<8, U2, C>, p.grid, lds, &a, s);
    case 16:
      if constexpr (U2 == 1) return coop_launch(fwd_vec_kernel<16, U2, C>, p.grid, lds, &a, s);
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_vec(const Plan& p, FwdArgs& a, hipStream_t s) {
  // exchange words a thread reads per step: 4*Hp/256 (at most 16)
  const bool wide = p.words_per_thread > 4;
  if (p.NJ == 8) return wide ? fwd_vec_l<1, 16>(p, a, s) : fwd_vec_l<1, 4>(p, a, s);
  return wide ? fwd_vec_l<2, 16>(p, a, s) : fwd_vec_l<2, 4>(p, a, s);
}

}  // namespace lstm
