// Mixed batch in one launch: prefill / extend sequences (several query rows)
// and decode sequences (one query row) together, as a serving step schedules
// them (Transformer 추론 커널 (3/10), §6 counts such a step's rows as
// M = 2 x 256 + 30 x 1).
//
// A decode row run as a prefill item would stream its whole context through
// one workgroup, one 64-key tile per step, while a decode range streams it
// 16 keys per step with every KV head of the block at once and cuts long
// contexts into pieces merged by log-sum-exp (§13, §16).  So the grid is
// shared: the first P workgroups walk the prefill items of the sequences with
// more than one query row (the persistent loop of prefill_impl.hpp, with P in
// place of the grid), the others cut the key blocks of the one-row sequences
// into equal ranges and merge the pieces in the same launch (the decode part
// of decode_impl.hpp).  The host cannot tell the two kinds apart without
// reading cu_seqlens_q, so every workgroup forms the same split from
// cu_seqlens_q and seqlens_k itself: P follows the two parts' estimated
// costs, in steps of 8 workgroups (one per XCD), and leaves the decode part
// enough ranges for its table window.
#include <atomic>

#include "decode_impl.hpp"
#include "prefill_impl.hpp"

namespace kvs {

// Estimated cost, in decode block-steps of one workgroup: a prefill step (a
// 64-key tile for the workgroup's query rows) takes about 1.4, and every item
// about two steps more for its set-up and epilogue (the weight that ended
// both parts closest together over mixed batches of 1-8 prompts and 30-63
// one-row sequences).
constexpr float kMixPrefillStep = 1.4f;

// NW waves per workgroup (4: two workgroups per CU; 8: one): the prefill
// part's waves and the decode part's KV heads per workgroup.
template <int D, bool WIN, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void mixed_kernel(AttnParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ float s_cpf[NW];
  __shared__ int s_dblk[NW];
  __shared__ int s_ntm[NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = (int)gridDim.x;
  const int nhg = p.Hkv / p.hpw;   // decode head groups (workgroups per range)
  const int TW = 32 * p.TPW;       // query rows per prefill item
  const int win = WIN ? p.window : 0;
  // ---- the split: the same arithmetic, in the same order, in every workgroup.
  // The same pass stages the batch metadata where the prefill part keeps it
  // and finds the most token tiles of any sequence (what the prefill part's
  // own set-up would do), so a prefill workgroup starts on its items at once.
  const bool staged = p.meta_lds != 0;
  int* s_cq = reinterpret_cast<int*>(smem + 2 * PCfg<D, true, NW>::STAGE);   // [B + 1]
  int* s_lk = s_cq + p.B + 1;                                              // [B]
  float cpf = 0.f;   // prefill part
  int dblk = 0;      // decode part: key blocks of the one-row sequences
  int ntm = 0;       // most token tiles of a sequence
  for (int b = tid; b < p.B; b += 64 * NW) {
    const int q0 = p.cu_q[b], q1 = p.cu_q[b + 1], lk = p.lens_k[b];
    const int Lq = q1 - q0;
    if (staged) {
      s_cq[b] = q0;
      s_lk[b] = lk;
      if (b == p.B - 1) s_cq[p.B] = q1;
    }
    ntm = max(ntm, (Lq + TW - 1) / TW);
    if (Lq == 1) {
      dblk += seq_blocks(lk, win);
    } else if (Lq > 1) {
      // token tiles t = 0 .. nt - 1 see (causally) up to cached + (t + 1) TW
      // keys, a sliding window at most win + TW of them
      const float nt = (float)((Lq + TW - 1) / TW);
      const float cached = (float)(lk - Lq);
      float keys = p.causal ? nt * cached + 0.5f * (float)TW * nt * (nt + 1.f) : nt * (float)lk;
      if (WIN) keys = fminf(keys, nt * (float)(win + TW));
      cpf += (float)p.NHG * kMixPrefillStep * (keys * (1.f / 64.f) + 2.f * nt);
    }
  }
  cpf = wave_sum(cpf);
  dblk = wave_inclusive_sum(dblk);   // lane 63 holds the wave's total
  ntm = (int)wave_max((float)ntm);
  if (lane == 63) {
    s_cpf[wave] = cpf;
    s_dblk[wave] = dblk;
    s_ntm[wave] = ntm;
  }
  __syncthreads();   // (also: the staged metadata is in place before either part starts)
  float cp = 0.f;
  int db = 0, nt = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    cp += s_cpf[i];
    db += s_dblk[i];
    nt = max(nt, s_ntm[i]);
  }
  nt = __builtin_amdgcn_readfirstlane(nt);
  cp = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(cp)));
  db = __builtin_amdgcn_readfirstlane(db);
  int P = W;   // no one-row sequence: the whole grid runs prefill items
  if (db > 0) {
    // decode workgroups a range's table window needs (the planner keeps
    // W >= 8 + this, so P >= 8 below)
    const int need = nhg * ((db + kDecodeTblWin - 1) / kDecodeTblWin);
    const int pmax = max(0, (W - need) / 8 * 8);
    const float cd = (float)db * (float)nhg;
    const int pe = (int)((float)W * cp / (cp + cd) + 4.f) / 8 * 8;
    P = cp > 0.f ? min(max(pe, 8), pmax) : 0;
  }
  const int w = (int)blockIdx.x;
  if (w < P) {
    prefill_body<D, true, NW, WIN, false>(p, P, w, nt);
  } else {
    const int nd = (W - P) / nhg;   // ranges per head group
    const int v = w - P;
    if (v < nd * nhg) decode_body<D, true, false, WIN, false, false, false, true>(p, v % nd, v / nd, nd);
  }
}

template <int D, bool WIN, int NW>
static hipError_t launch_mixed_t(const AttnParams& p, int grid, size_t lds, hipStream_t s) {
  const void* kern = reinterpret_cast<const void*>(&mixed_kernel<D, WIN, NW>);
  // dynamic LDS above the default limit must be requested; grow it as needed
  // (per instantiation; atomic so that concurrent first calls are safe)
  static std::atomic<size_t> lds_granted{0};
  if (lds > lds_granted.load(std::memory_order_relaxed)) {
    const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) {
      (void)hipGetLastError();  // do not leave the error for the caller's next HIP call
      return e;
    }
    size_t cur = lds_granted.load(std::memory_order_relaxed);
    while (cur < lds && !lds_granted.compare_exchange_weak(cur, lds, std::memory_order_relaxed)) {
    }
  }
  hipLaunchKernelGGL((mixed_kernel<D, WIN, NW>), dim3(grid), dim3(64 * NW), lds, s, p);
  return hipGetLastError();
}

template <int NW>
static hipError_t launch_mixed_n(const AttnParams& p, int D, int grid, size_t lds, hipStream_t s) {
  if (p.window > 0) return D == 64 ? launch_mixed_t<64, true, NW>(p, grid, lds, s) : launch_mixed_t<128, true, NW>(p, grid, lds, s);
  return D == 64 ? launch_mixed_t<64, false, NW>(p, grid, lds, s) : launch_mixed_t<128, false, NW>(p, grid, lds, s);
}

hipError_t launch_mixed(const AttnParams& p, int D, int grid, size_t lds, hipStream_t s) {
  if (p.pnw == 4) return launch_mixed_n<4>(p, D, grid, lds, s);
  if (p.pnw == 8) return launch_mixed_n<8>(p, D, grid, lds, s);
  return hipErrorInvalidValue;
}

}  // namespace kvs
