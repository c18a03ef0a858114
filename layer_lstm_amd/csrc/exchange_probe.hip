// exchange_probe.hip -- the per-step exchange of the persistent forward
// recurrence with nothing else in the step: the floor under its step time.
//
// A step of the forward recurrence (recurrent.hip) is: wait for the step
// flags of every work-group of the batch group, copy the group's rows of
// h_{t-1} from the exchange ring into LDS, the product and the gate math,
// then write this work-group's units of h_t into the next ring slot, wait for
// those stores and set the step flag.  The probe keeps the waits, the copy,
// the stores and the flag -- with the same layout (grid, batch groups, rows
// and units per work-group, XCD-local or spread), the same ring and flag
// addresses and the same load and store kinds -- and drops the product and
// the gate math.  Its time per step is what any step of that layout costs
// before arithmetic; lstm_probe_exchange reports it.
#include "recurrent_common.hpp"

namespace lstm {

struct ProbeArgs {
  void* HD;          // [2][Bp][Hp] ring of E-byte elements
  uint32_t* HF;      // [nBG][nJG] step flags
  uint32_t hd_bytes;
  uint32_t* err;
  int T, B, H, NB, NJ, nJG, Hp, Bp, nBG, nxcd, local, E;
};

template <int NW>
__global__ void __launch_bounds__(64 * NW, 1) exchange_probe_kernel(ProbeArgs a) {
  constexpr int NTH = 64 * NW;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bg, jg;
  take_role(blockIdx.x, a.nBG, a.nJG, a.nxcd, a.local, 0, bg, jg);
  const bool local = a.local != 0;
  const int b0 = bg * a.NB, j0 = jg * a.NJ;
  const int NBv = (a.B - b0) < a.NB ? (a.B - b0) : a.NB;
  const int rowB = a.Hp * a.E, strideH = rowB + 16;
  const int cpr = (a.H * a.E + 15) / 16, nchunk = NBv * cpr;
  const bool dma = (a.H * a.E) % 1024 == 0;
  const __amdgpu_buffer_rsrc_t hd_rsrc = make_rsrc(a.HD, a.hd_bytes);
  const uint32_t hl_lds = (uint32_t)(uintptr_t)(lds_void_t*)smem;
  bool dead = false;
  for (int t = 0; t < a.T; ++t) {
    if (t > 0 && tid < a.nJG) wait_flag(a.HF + bg * a.nJG + tid, (uint32_t)t, a.err, dead);
    __syncthreads();
    if (t > 0) {
      const uint32_t slot0 = (uint32_t)(((t - 1) & 1) * a.Bp + b0) * (uint32_t)rowB;
      if (dma) {
        for (int j = w; j * 64 < nchunk; j += NW) {
          const int bl = (64 * j) / cpr, cc = 64 * j - bl * cpr;
          lds_dma16_at<true>(hd_rsrc, hl_lds + (uint32_t)(bl * strideH + cc * 16),
                             slot0 + (uint32_t)(bl * rowB + lane * 16), (uint32_t)(cc * 16));
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      } else {
        for (int q = tid; q < nchunk; q += NTH) {
          const int bl = q / cpr, cc = q - bl * cpr;
          *(u32x4_t*)(smem + bl * strideH + cc * 16) = load16_coherent(hd_rsrc, slot0 + (uint32_t)(bl * rowB + cc * 16));
        }
      }
      __builtin_amdgcn_s_barrier();
    }
    // this work-group's units of the next slot: NB rows x NJ units
    char* dst = (char*)a.HD + (int64_t)(t & 1) * a.Bp * rowB;
    for (int e = tid; e < NBv * a.NJ; e += NTH) {
      const int bl = e / a.NJ, u = j0 + e % a.NJ;
      if (u >= a.H) continue;
      char* p = dst + (int64_t)(b0 + bl) * rowB + (int64_t)u * a.E;
      if (a.E == 2)
        store_elem<uint16_t>((uint16_t*)p, (uint16_t)(t + u), local);
      else
        store_elem<uint32_t>((uint32_t*)p, (uint32_t)(t + u), local);
    }
    wait_vmem();
    __syncthreads();
    if (tid == 0) store_flag(a.HF + bg * a.nJG + jg, (uint32_t)(t + 1), local);
  }
}

hipError_t launch_exchange_probe(const Plan& p, void* HX, uint32_t* err, hipStream_t s) {
  char* hd = (char*)HX;
  ProbeArgs a{hd, (uint32_t*)(hd + p.off_hflags), (uint32_t)p.off_hflags, err, (int)p.T, (int)p.B, (int)p.H,
              p.NB, p.NJ, p.nJG, p.Hp, p.Bp, p.nBG, p.nxcd, p.xcd_local, p.esize};
  const size_t lds = (size_t)(p.NB < 16 ? 16 : p.NB) * (p.Hp * p.esize + 16);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  if (p.waves == 8) return coop_launch(exchange_probe_kernel<8>, p.grid, lds, &a, s, 512);
  return coop_launch(exchange_probe_kernel<kWaves>, p.grid, lds, &a, s, kRecThreads);
}

}  // namespace lstm
